"""Calls on a stream other than the current one.

The binding allocates a call's temporaries (the long-row split workspace,
default outputs) on the stream the call runs on.  Here a causal forward with
rows longer than 128 key blocks runs on a side stream held back by a bounded
spin kernel, and its binding-owned workspace is dropped on return; meanwhile
the default stream allocates memory of the same size and overwrites it.  If
the workspace were owned by the default stream, that memory could be the
workspace the side stream's kernels are about to use.  The result must equal,
bit for bit, the same call made on the default stream alone."""
import numpy as np
import pytest
import torch

import block_sparse_attention_amd as bsa
from block_sparse_attention_amd import inputs as gen
from oracle import attention as oa
from tests.gpu_util import check_close, gpu_bf16_to_f64, say, to_gpu, to_gpu_bf16

pytestmark = pytest.mark.gpu


def _delay(stream):
    """Queue about 20 ms of bounded GPU work on `stream`."""
    with torch.cuda.stream(stream):
        if hasattr(torch.cuda, "_sleep"):
            torch.cuda._sleep(40_000_000)
        else:  # pragma: no cover
            a = torch.ones((4096, 4096), device="cuda")
            for _ in range(20):
                a = a @ a * 1e-4


@pytest.mark.parametrize("D", [64, 128])
def test_split_rows_on_a_side_stream(D):
    rng = np.random.default_rng(11 + D)
    B, H, S = 1, 2, 8400
    nb = -(-S // 64)
    x = {n: gen.f32_to_bf16_bits(rng.standard_normal((B, H, S, D), dtype=np.float32))
         for n in ("q", "k", "v")}
    mask = (rng.random((B, H, nb, nb)) < 0.3).astype(np.uint8)
    mask[..., nb - 4:, :] = 1
    mask[..., np.arange(nb), np.arange(nb)] = 1
    q, k, v = (to_gpu_bf16(x[n]) for n in ("q", "k", "v"))
    m = to_gpu(mask)
    need = bsa.bsattn_fwd_workspace_bytes(B, H, S, D)
    say(f"[streams] side-stream split forward D={D} workspace={need}")
    ref = bsa.bsattn_fwd(q, k, v, m, True)
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):
        _delay(side)
        out = torch.empty_like(q)
        out.record_stream(side)
        bsa.bsattn_fwd(q, k, v, m, True, out=out, stream=side)   # workspace: binding-owned
        # the default stream reuses freed memory at once and overwrites it
        junk = torch.empty(need, dtype=torch.uint8, device="cuda")
        junk.fill_(0xFF)
        outs.append(out)
        del junk
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o.view(torch.int16), ref.view(torch.int16))
    rows = list(range(64 * (nb - 4), S, 7)) + [0, 4095]
    f = {n: gen.bf16_bits_to_f64(x[n]) for n in ("q", "k", "v")}
    want = np.stack([oa.prefill_head_rows(f["q"][0, h], f["k"][0, h], f["v"][0, h], mask[0, h], True, rows)
                     for h in range(H)])
    check_close(gpu_bf16_to_f64(outs[-1])[0][:, rows], want, f"side stream D{D}")
