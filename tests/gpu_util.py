"""Helpers for the GPU parity tests (host-side marshalling and comparison)."""
import sys

import numpy as np

from block_sparse_attention_amd import inputs as gen

MAX_ABS = 1e-2     # output tolerance: max |gpu - oracle| (bf16 inputs, fp32 accumulation)
MEAN_ABS = 1e-3    # output tolerance: mean |gpu - oracle|


def say(msg: str) -> None:
    """Name the case before a GPU step, so a fault can be attributed."""
    print(msg, flush=True)
    sys.stdout.flush()


def to_gpu_bf16(bits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda")


def to_gpu(arr: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(arr)).to("cuda")


def gpu_bf16_to_f64(t) -> np.ndarray:
    import torch
    bits = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return gen.bf16_bits_to_f64(bits)


def check_close(got: np.ndarray, want: np.ndarray, what: str, max_abs=MAX_ABS, mean_abs=MEAN_ABS):
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - want)
    mx, mn = float(err.max()) if err.size else 0.0, float(err.mean()) if err.size else 0.0
    say(f"  {what}: max_abs={mx:.3e} mean_abs={mn:.3e}")
    assert mx <= max_abs, f"{what}: max abs err {mx} > {max_abs}"
    assert mn <= mean_abs, f"{what}: mean abs err {mn} > {mean_abs}"
    return mx, mn


def parallel_map(fn, items, workers: int = 8):
    """fn over items on a thread pool (numpy releases the GIL in its array
    loops), BLAS single-threaded in each worker; results in item order."""
    import concurrent.futures as cf
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(limits=1, user_api="blas")
    except Exception:  # pragma: no cover
        limit = None
    try:
        with cf.ThreadPoolExecutor(max_workers=workers) as ex:
            return list(ex.map(fn, items))
    finally:
        if limit is not None and hasattr(limit, "restore_original_limits"):
            limit.restore_original_limits()
