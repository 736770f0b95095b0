"""C-ABI boundary checks that need no GPU: the library loads, exports every
function the header declares, and rejects bad arguments on the host before
any launch.  Also pins the library's split heuristic against the oracle's."""
import ctypes
import os
import re

import pytest

import block_sparse_attention_amd as bsa
from oracle import heuristic as oh

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsattn.h")


def _lib():
    if not os.path.exists(bsa.LIB_PATH):
        pytest.skip("libbsattn.so not built (run __graft_entry__.build())")
    return bsa.load_library()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bsattn_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_binding_names():
    assert set(_declared()) == set(bsa.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    lib = _lib()
    for name in _declared():
        assert hasattr(lib, name), name
    assert bsa.bsattn_version().count(".") == 2
    for s in range(6):
        assert bsa.bsattn_status_string(s)


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every case below fails validation first


def test_mask_builders_validate_on_host():
    lib = _lib()
    assert lib.bsattn_build_mask_topk(None, 1, 1, 4, 2, 0, 1, FAKE, None) == 1
    assert lib.bsattn_build_mask_topk(FAKE, 1, 1, 4, 5, 0, 1, FAKE, None) == 2   # topk > nb
    assert lib.bsattn_build_mask_topk(FAKE, 1, 1, 4, -1, 0, 1, FAKE, None) == 2
    assert lib.bsattn_build_mask_topk(FAKE, 0, 1, 4, 1, 0, 1, FAKE, None) == 2
    assert lib.bsattn_build_mask_threshold(FAKE, 1, 1, 0, 0.5, 0, 1, FAKE, None) == 2
    assert lib.bsattn_build_mask_threshold(FAKE, 1, 1, 4, 0.5, 0, 1, None, None) == 1
    # more than 2^31 - 1 rows
    assert lib.bsattn_build_mask_topk(FAKE, 65536, 65536, 1, 1, 0, 1, FAKE, None) == 2
    assert lib.bsattn_build_mask_threshold(FAKE, 65536, 65536, 1, 0.5, 0, 1, FAKE, None) == 2
    assert lib.bsattn_mask_to_indices(FAKE, 65536, 65536, 4, 1, FAKE, FAKE, None) == 2
    assert lib.bsattn_mask_to_indices(FAKE, 1, -1, 4, 1, FAKE, FAKE, None) == 2
    assert lib.bsattn_mask_to_indices(FAKE, 1, 1, 4, 1, None, FAKE, None) == 1


def test_fwd_validates_on_host():
    lib = _lib()
    F = FAKE
    assert lib.bsattn_fwd(F, F, None, F, 1, 1, 64, 64, 1, F, None, 0, None) == 1
    assert lib.bsattn_fwd(F, F, F, F, 1, 1, 0, 64, 1, F, None, 0, None) == 2
    assert lib.bsattn_fwd(F, F, F, F, 1, 1, 64, 96, 1, F, None, 0, None) == 3
    assert lib.bsattn_fwd(F, F, F, F, 1, 1, 64, 256, 1, F, None, 0, None) == 3
    assert lib.bsattn_fwd_indices(F, F, F, None, F, 1, 1, 64, 64, 1, F, None) == 1
    assert lib.bsattn_fwd_indices(F, F, F, F, F, 1, 1, 64, 32, 1, F, None) == 3
    assert lib.bsattn_fwd_workspace_bytes(2, 16, 4096, 64) == 0


def test_fwd_long_row_workspace_on_host():
    """Causal rows past 128 key blocks split in two through the workspace."""
    lib = _lib()
    F = FAKE
    S = 8320                       # 130 key blocks: query blocks 128 and 129 can split
    need = lib.bsattn_fwd_workspace_bytes(1, 8, S, 128)
    slots = 8 * 2
    assert need >= slots * (2 * 64 * 128 * 4 + 2 * 64 * 8 + 4) and need % 256 == 0
    assert lib.bsattn_fwd_workspace_bytes(1, 8, S, 64) < need      # halves of D = 64 rows
    assert lib.bsattn_fwd(F, F, F, F, 1, 8, S, 128, 1, F, None, 0, None) == 4
    assert lib.bsattn_fwd(F, F, F, F, 1, 8, S, 128, 1, F, F, need - 1, None) == 4
    misaligned = ctypes.c_void_p(0x1008)
    assert lib.bsattn_fwd(F, F, F, F, 1, 8, S, 128, 1, F, misaligned, need, None) == 4
    assert lib.bsattn_fwd_workspace_bytes(1, 8, 8192, 128) == 0    # 128 blocks: no row can exceed 128
    assert lib.bsattn_fwd_workspace_bytes(1, 8, 8193, 128) > 0
    assert lib.bsattn_fwd_workspace_bytes(0, 8, S, 128) == 0
    assert lib.bsattn_fwd_workspace_bytes(1, 8, S, 96) == 0
    # beyond 2 GiB the long rows run unsplit and no workspace is asked for
    assert lib.bsattn_fwd_workspace_bytes(64, 64, 65536, 128) == 0


def test_decode_validates_on_host():
    lib = _lib()
    F = FAKE
    args = dict(B=2, Hq=8, Hkv=2, D=128, ms=4, tk=100, ns=2)

    def call(q=F, cu=F, B=2, Hq=8, Hkv=2, D=128, Dv=128, ms=4, tk=100, ns=2, ws=None, wsb=0):
        return lib.bsattn_decode_gqa(q, F, F, cu, F, B, Hq, Hkv, D, Dv, ms, tk, ns, F, ws, wsb, None)

    assert call(q=None) == 1
    assert call(cu=None) == 1
    assert call(Hq=6, Hkv=4) == 2          # Hq % Hkv
    assert call(ns=5) == 2                 # more splits than slots
    assert call(ms=0) == 2
    assert call(tk=0) == 2
    assert call(D=80) == 3
    assert call(Dv=96) == 3
    assert call(Hq=130, Hkv=2) == 3        # group of 65 query heads
    assert call(Hq=128, Hkv=2, ns=2) == 4  # a group of 64 is taken; partials need a workspace
    assert call(D=64, Dv=128, ns=2) == 4   # head dims may differ
    assert call(ns=2) == 4                 # partials need a workspace
    need = lib.bsattn_decode_workspace_bytes(2, 8, 128, 2)
    assert need >= 2 * 8 * 2 * (128 + 1) * 4 and need % 256 == 0
    assert call(ns=2, ws=F, wsb=need - 1) == 4
    assert lib.bsattn_decode_workspace_bytes(2, 8, 128, 1) == 0    # one split writes the output directly
    assert lib.bsattn_decode_workspace_bytes(0, 8, 128, 2) == 0


def test_noalloc_decode_validates_on_host():
    lib = _lib()
    F = FAKE

    def call(q=F, cu=F, B=2, Hq=8, Hkv=2, D=128, Dv=128, ms=4, tk=100, ns=2):
        return lib.bsattn_decode_gqa_noalloc(q, F, F, cu, F, B, Hq, Hkv, D, Dv, ms, tk, ns, F, None)

    assert lib.bsattn_decode_noalloc_scratch_bytes() == 8 << 20
    assert call(q=None) == 1
    assert call(cu=None) == 1
    assert call(Hq=6, Hkv=4) == 2
    assert call(ns=5) == 2
    assert call(tk=0) == 2
    assert call(D=80) == 3
    # partials beyond the 8 MiB scratch array are refused before any device call
    assert lib.bsattn_decode_workspace_bytes(64, 64, 128, 64) > 8 << 20
    assert call(B=64, Hq=64, Hkv=4, ms=64, ns=64) == 4


def test_fused_fwd_validates_on_host():
    lib = _lib()
    F = FAKE
    assert lib.bsattn_fwd_topk(None, F, F, F, 1, 1, 256, 64, 2, 0, 1, 1, None, F, None, 0, None) == 1
    assert lib.bsattn_fwd_topk(F, F, F, None, 1, 1, 256, 64, 2, 0, 1, 1, None, F, None, 0, None) == 1
    assert lib.bsattn_fwd_topk(F, F, F, F, 1, 1, 256, 64, 5, 0, 1, 1, None, F, None, 0, None) == 2   # topk > nb
    assert lib.bsattn_fwd_topk(F, F, F, F, 1, 1, 256, 64, -1, 0, 1, 1, None, F, None, 0, None) == 2
    assert lib.bsattn_fwd_topk(F, F, F, F, 1, 1, 256, 96, 2, 0, 1, 1, None, F, None, 0, None) == 3
    assert lib.bsattn_fwd_topk(F, F, F, F, 1, 1, 64 * 257, 64, 2, 0, 1, 1, None, F, None, 0, None) == 3
    assert lib.bsattn_fwd_threshold(F, F, F, F, 1, 1, 64 * 257, 64, 0.5, 0, 1, 1, None, F, None, 0, None) == 3
    assert lib.bsattn_fwd_threshold(F, F, F, None, 1, 1, 256, 64, 0.5, 0, 1, 1, None, F, None, 0, None) == 1
    assert lib.bsattn_fwd_threshold(F, F, F, F, 0, 1, 256, 64, 0.5, 0, 1, 1, None, F, None, 0, None) == 2
    # long causal rows split as in bsattn_fwd, so the same workspace is required
    S = 8320
    need = lib.bsattn_fwd_workspace_bytes(1, 8, S, 128)
    assert lib.bsattn_fwd_topk(F, F, F, F, 1, 8, S, 128, 2, 0, 1, 1, None, F, None, 0, None) == 4
    assert lib.bsattn_fwd_threshold(F, F, F, F, 1, 8, S, 128, 0.5, 0, 1, 1, None, F, F, need - 1,
                                    None) == 4
    misaligned = ctypes.c_void_p(0x1008)
    assert lib.bsattn_fwd_topk(F, F, F, F, 1, 8, S, 128, 2, 0, 1, 1, None, F, misaligned, need,
                               None) == 4
    # past 256 key blocks the fused forms run as builder + forward through mask_out; every
    # check (mask_out present, workspace, shapes) still comes before the first launch
    S2 = 64 * 260
    need2 = lib.bsattn_fwd_workspace_bytes(1, 2, S2, 64)
    assert need2 > 0
    assert lib.bsattn_fwd_topk(F, F, F, F, 1, 2, S2, 64, 2, 0, 1, 1, None, F, F, need2, None) == 3
    assert lib.bsattn_fwd_topk(F, F, F, F, 1, 2, S2, 64, 2, 0, 1, 1, F, F, None, 0, None) == 4
    assert lib.bsattn_fwd_threshold(F, F, F, F, 1, 2, S2, 64, 0.5, 0, 1, 1, F, F, F, need2 - 1,
                                    None) == 4
    assert lib.bsattn_fwd_threshold(F, F, F, F, 1, 2, S2, 96, 0.5, 0, 1, 1, F, F, None, 0,
                                    None) == 3
    assert lib.bsattn_fwd_topk(F, F, F, F, 1, 2, S2, 64, 261, 0, 1, 1, F, F, F, need2, None) == 2


def test_xattn_validates_on_host():
    lib = _lib()
    F = FAKE
    ws = 1 << 40   # claimed size: no call below gets past validation
    # block sums: q k B H Sq Sk D stride norm causal out ws ws_bytes stream
    assert lib.bsattn_xattn_block_sums(None, F, 1, 1, 256, 256, 64, 8, 1.0, 1, F, F, ws, None) == 1
    assert lib.bsattn_xattn_block_sums(F, F, 1, 1, 256, 256, 64, 8, 1.0, 1, None, F, ws, None) == 1
    assert lib.bsattn_xattn_block_sums(F, F, 1, 1, 256, 128, 64, 8, 1.0, 1, F, F, ws, None) == 2   # Sk < Sq
    assert lib.bsattn_xattn_block_sums(F, F, 1, 1, 100, 100, 64, 8, 1.0, 1, F, F, ws, None) == 2   # S % stride
    assert lib.bsattn_xattn_block_sums(F, F, 1, 1, 128, 160, 64, 8, 1.0, 1, F, F, ws, None) == 2   # (Sk-Sq) % 64
    assert lib.bsattn_xattn_block_sums(F, F, 1, 1, 256, 256, 64, 8, 0.0, 1, F, F, ws, None) == 2   # norm
    assert lib.bsattn_xattn_block_sums(F, F, 1, 1, 256, 256, 64, 8, float("inf"), 1, F, F, ws, None) == 2
    assert lib.bsattn_xattn_block_sums(F, F, 1, 1, 256, 256, 96, 8, 1.0, 1, F, F, ws, None) == 3   # D
    assert lib.bsattn_xattn_block_sums(F, F, 1, 1, 256, 256, 64, 2, 1.0, 1, F, F, ws, None) == 3   # stride
    assert lib.bsattn_xattn_block_sums(F, F, 1, 1, 64, 64 * 1025, 64, 8, 1.0, 1, F, F, ws, None) == 3
    need = lib.bsattn_xattn_workspace_bytes(1, 2, 256, 512, 8)
    assert need >= 2 * (256 // 8) * 8 * 4 + 2 * 4 * 8 * 4
    assert lib.bsattn_xattn_workspace_bytes(1, 2, 256, 100, 8) == 0
    assert lib.bsattn_xattn_block_sums(F, F, 1, 2, 256, 512, 64, 8, 1.0, 1, F, F, need - 1, None) == 4
    assert lib.bsattn_xattn_block_sums(F, F, 1, 2, 256, 512, 64, 8, 1.0, 1, F, None, need, None) == 4
    # cumulative selection: sums B H nbq nbk thr sink diag causal mask stream
    assert lib.bsattn_build_mask_cumulative(None, 1, 1, 2, 2, 0.9, 1, 1, 1, F, None) == 1
    assert lib.bsattn_build_mask_cumulative(F, 1, 1, 2, 2, 0.9, 1, 1, 1, None, None) == 1
    assert lib.bsattn_build_mask_cumulative(F, 1, 1, 3, 2, 0.9, 1, 1, 1, F, None) == 2
    assert lib.bsattn_build_mask_cumulative(F, 0, 1, 2, 2, 0.9, 1, 1, 1, F, None) == 2
    assert lib.bsattn_build_mask_cumulative(F, 1, 1, 2, 1025, 0.9, 1, 1, 1, F, None) == 3
    # the whole estimator
    assert lib.bsattn_xattn_estimate(F, F, 1, 1, 256, 256, 64, 8, 1.0, 0.9, 1, 1, 1, None, None, F, ws, None) == 1
    assert lib.bsattn_xattn_estimate(F, F, 1, 1, 256, 256, 64, 4 * 3, 1.0, 0.9, 1, 1, 1, None, F, F, ws, None) == 2
    assert lib.bsattn_xattn_estimate(F, F, 1, 1, 256, 256, 64, 8, 1.0, 0.9, 1, 1, 1, None, F, F, 16, None) == 4


def test_chunk_fwd_validates_on_host():
    lib = _lib()
    F = FAKE
    assert lib.bsattn_fwd_chunk(None, F, F, F, 1, 1, 64, 128, 64, 1, F, None) == 1
    assert lib.bsattn_fwd_chunk(F, F, F, None, 1, 1, 64, 128, 64, 1, F, None) == 1
    assert lib.bsattn_fwd_chunk(F, F, F, F, 1, 1, 129, 128, 64, 1, F, None) == 2   # Sq > Sk
    assert lib.bsattn_fwd_chunk(F, F, F, F, 1, 1, 0, 128, 64, 1, F, None) == 2
    assert lib.bsattn_fwd_chunk(F, F, F, F, 0, 1, 64, 128, 64, 1, F, None) == 2
    assert lib.bsattn_fwd_chunk(F, F, F, F, 1, 1, 64, 128, 96, 1, F, None) == 3


def test_fwd_key_block_limit_on_host():
    """The longest key range each head dim takes: every forward form refuses
    one block more before any launch (UNSUPPORTED)."""
    lib = _lib()
    F = FAKE
    assert lib.bsattn_fwd_max_key_blocks(96) == 0
    m64, m128 = lib.bsattn_fwd_max_key_blocks(64), lib.bsattn_fwd_max_key_blocks(128)
    assert 256 < m128 < m64 <= 65535, (m64, m128)   # D = 128 holds a larger K/V ring
    for D, m in ((64, m64), (128, m128)):
        Sk = (m + 1) * 64
        assert lib.bsattn_fwd_chunk(F, F, F, F, 1, 1, 64, Sk, D, 1, F, None) == 3
        assert lib.bsattn_fwd_chunk(F, F, F, F, 1, 1, 64, Sk - 63, D, 0, F, None) == 3  # ragged tail
        assert lib.bsattn_fwd(F, F, F, F, 1, 1, Sk, D, 0, F, None, 0, None) == 3
        assert lib.bsattn_fwd_indices(F, F, F, F, F, 1, 1, Sk, D, 0, F, None) == 3


def test_mask_form_decode_validates_on_host():
    lib = _lib()
    F = FAKE

    def call(q=F, bm=F, B=2, Hq=8, Hkv=2, D=128, Dv=128, nbk=4, tk=100, ns=2, ws=None, wsb=0):
        return lib.bsattn_decode_gqa_mask(q, F, F, F, bm, B, Hq, Hkv, D, Dv, nbk, tk, ns, F, ws, wsb,
                                          None)

    assert call(q=None) == 1
    assert call(bm=None) == 1
    assert call(nbk=0) == 2
    assert call(ns=5) == 2                 # more splits than mask columns
    assert call(tk=0) == 2
    assert call(Hq=6, Hkv=4) == 2
    assert call(D=96) == 3
    assert call(Dv=32) == 3
    assert call(Hq=130, Hkv=2) == 3
    assert call(ns=2) == 4


def test_paged_decode_validates_on_host():
    lib = _lib()
    F = FAKE

    def call(q=F, tab=F, B=2, Hq=8, Hkv=2, D=128, Dv=128, npg=16, psz=256, mbps=4, ms=8, ns=2,
             ws=None, wsb=0):
        return lib.bsattn_decode_gqa_paged(q, F, F, F, tab, F, B, Hq, Hkv, D, Dv, npg, psz, mbps, ms,
                                           ns, F, ws, wsb, None)

    assert call(q=None) == 1
    assert call(tab=None) == 1
    assert call(psz=96) == 2               # page size not a multiple of 64
    assert call(psz=0) == 2
    assert call(npg=0) == 2
    assert call(mbps=0) == 2
    assert call(ms=0) == 2
    assert call(ns=9) == 2
    assert call(Hq=130, Hkv=2) == 3
    assert call(Dv=80) == 3
    assert call(ns=2) == 4


def test_library_heuristic_matches_oracle_sweep():
    _lib()
    n = 0
    for B in (1, 2, 3, 8, 16, 64):
        for Hkv in (1, 2, 8):
            for G in (1, 4, 16):
                for ms in (1, 3, 4, 5, 17, 64, 200):
                    for cus in (80, 132, 256, 304):
                        want = oh.decode_num_splits(B, Hkv * G, Hkv, ms, 128, cus)
                        got = bsa.bsattn_decode_num_splits(B, Hkv * G, Hkv, ms, 128, cus)
                        assert got == want, (B, Hkv, G, ms, cus)
                        n += 1
    assert n > 1000
    assert bsa.bsattn_decode_num_splits(8, 32, 8, 64, 128, 256) == 4
    assert bsa.bsattn_decode_num_splits(8, 30, 8, 64, 128, 256) == 0   # Hq % Hkv


def test_binding_refuses_host_tensors():
    import torch
    _lib()
    q = torch.zeros((1, 1, 64, 64), dtype=torch.bfloat16)
    m = torch.ones((1, 1, 1, 1), dtype=torch.uint8)
    with pytest.raises(ValueError, match="GPU"):
        bsa.bsattn_fwd(q, q, q, m)
    with pytest.raises(ValueError, match="GPU"):
        bsa.bsattn_build_mask_topk(torch.zeros((1, 1, 2, 2)), 1)


C_PROGRAM = r"""
#include <stdio.h>
#include "bsattn.h"

/* A C99 caller of the ABI: every call below fails validation on the host,
   so no device memory is needed; the split heuristic is plain host code. */
int main(void) {
  const uint16_t* f16 = (const uint16_t*)0x1000;   /* never dereferenced */
  const float* f32 = (const float*)0x1000;
  uint8_t* m8 = (uint8_t*)0x1000;
  int bad = 0;
  bad += bsattn_build_mask_topk(NULL, 1, 1, 4, 2, 0, 1, m8, NULL) != BSATTN_ERR_NULL;
  bad += bsattn_build_mask_topk(f32, 1, 1, 4, 5, 0, 1, m8, NULL) != BSATTN_ERR_SHAPE;
  bad += bsattn_fwd(f16, f16, f16, m8, 1, 1, 64, 96, 1, (uint16_t*)f16, NULL, 0, NULL)
         != BSATTN_ERR_UNSUPPORTED;
  bad += bsattn_decode_num_splits(8, 32, 8, 64, 128, 256) != 4;
  bad += bsattn_decode_gqa(f16, f16, f16, NULL, NULL, 8, 32, 8, 128, 64, 64, 100, 4,
                           (uint16_t*)f16, NULL, 0, NULL) != BSATTN_ERR_NULL;
  printf("%s %s %d\n", bsattn_version(), bsattn_status_string(BSATTN_ERR_SHAPE), bad);
  return bad;
}
"""


def test_c_program_compiles_links_and_calls_the_abi(tmp_path):
    """The header is plain C99 and the library links and runs from C."""
    import shutil
    import subprocess
    _lib()
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "caller.c"
    exe = tmp_path / "caller"
    src.write_text(C_PROGRAM)
    libdir = os.path.dirname(bsa.LIB_PATH)
    r = subprocess.run([cc, "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                        str(src), "-o", str(exe), f"-L{libdir}", "-l:libbsattn.so",
                        f"-Wl,-rpath,{libdir}"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, (r.stdout, r.stderr)
    words = r.stdout.split()
    assert words[0] == bsa.bsattn_version() and words[-1] == "0", r.stdout
