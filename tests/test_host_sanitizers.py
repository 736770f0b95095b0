"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

api.hip (every entry point's argument checks, the workspace-size arithmetic
and the decode split heuristic) is compiled with the host-side sanitizers
only (-Xarch_host: the device code is built as in the normal library) and
linked with the normally built kernels into a scratch library.  A C harness
built with the same sanitizers drives every host-only path: each entry point
with each kind of bad argument (nothing reaches a launch, so no GPU is
needed), the size functions over small, large and overflowing arguments,
and the split heuristic over a grid.  Any sanitizer report fails the run.
CPU only."""
import os
import shutil
import subprocess

import pytest

import block_sparse_attention_amd as bsa
from block_sparse_attention_amd import build as bld

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"

HARNESS = r"""
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include "bsattn.h"

#define CHECK(expr, want)                                                     \
  do {                                                                        \
    int got_ = (int)(expr);                                                   \
    if (got_ != (int)(want)) {                                                \
      printf("line %d: %s = %d, want %d\n", __LINE__, #expr, got_, (int)(want)); \
      bad++;                                                                  \
    }                                                                         \
  } while (0)

int main(void) {
  int bad = 0;
  const uint16_t* h = (const uint16_t*)0x1000;   /* never dereferenced */
  uint16_t* ho = (uint16_t*)0x1000;
  const float* f = (const float*)0x1000;
  float* fo = (float*)0x1000;
  uint8_t* m = (uint8_t*)0x1000;
  const int32_t* ci = (const int32_t*)0x1000;
  int32_t* io = (int32_t*)0x1000;
  void* ws = (void*)0x1000;
  const int big = 0x7fffffff;

  for (int s = -1; s <= 6; ++s) if (!bsattn_status_string((bsattn_status)s)) bad++;
  if (!bsattn_version()) bad++;

  /* mask builders and compaction */
  CHECK(bsattn_build_mask_topk(NULL, 1, 1, 4, 2, 0, 1, m, NULL), BSATTN_ERR_NULL);
  CHECK(bsattn_build_mask_topk(f, 1, 1, 4, 5, 0, 1, m, NULL), BSATTN_ERR_SHAPE);
  CHECK(bsattn_build_mask_topk(f, big, big, big, 1, 0, 1, m, NULL), BSATTN_ERR_SHAPE);
  CHECK(bsattn_build_mask_threshold(f, 0, 1, 4, 0.5f, 0, 1, m, NULL), BSATTN_ERR_SHAPE);
  CHECK(bsattn_mask_to_indices(m, 1, 1, 4, 1, NULL, io, NULL), BSATTN_ERR_NULL);
  CHECK(bsattn_mask_to_indices(m, big, big, big, 1, io, io, NULL), BSATTN_ERR_SHAPE);

  /* forward forms */
  CHECK(bsattn_fwd(h, h, NULL, m, 1, 1, 64, 64, 1, ho, NULL, 0, NULL), BSATTN_ERR_NULL);
  CHECK(bsattn_fwd(h, h, h, m, 1, 1, 0, 64, 1, ho, NULL, 0, NULL), BSATTN_ERR_SHAPE);
  CHECK(bsattn_fwd(h, h, h, m, 1, 1, 64, 96, 1, ho, NULL, 0, NULL), BSATTN_ERR_UNSUPPORTED);
  CHECK(bsattn_fwd(h, h, h, m, big, big, big, 128, 0, ho, NULL, 0, NULL), BSATTN_ERR_SHAPE);
  CHECK(bsattn_fwd(h, h, h, m, 1, 8, 8320, 128, 1, ho, NULL, 0, NULL), BSATTN_ERR_WORKSPACE);
  CHECK(bsattn_fwd(h, h, h, m, 1, 8, 8320, 128, 1, ho, (void*)0x1008, (size_t)1 << 40, NULL),
        BSATTN_ERR_WORKSPACE);
  CHECK(bsattn_fwd_indices(h, h, h, NULL, ci, 1, 1, 64, 64, 1, ho, NULL), BSATTN_ERR_NULL);
  CHECK(bsattn_fwd_chunk(h, h, h, m, 1, 1, 128, 64, 64, 1, ho, NULL), BSATTN_ERR_SHAPE);
  CHECK(bsattn_fwd_chunk(h, h, h, m, 1, 1, 64, 64 * 70000, 64, 1, ho, NULL),
        BSATTN_ERR_UNSUPPORTED);
  CHECK(bsattn_fwd_topk(h, h, h, f, 1, 1, 256, 64, 5, 0, 1, 1, NULL, ho, NULL, 0, NULL),
        BSATTN_ERR_SHAPE);
  CHECK(bsattn_fwd_topk(h, h, h, f, 1, 2, 64 * 260, 64, 2, 0, 1, 1, NULL, ho, ws, 1 << 30, NULL),
        BSATTN_ERR_UNSUPPORTED);
  CHECK(bsattn_fwd_threshold(h, h, h, f, 1, 2, 64 * 260, 64, 0.5f, 0, 1, 1, m, ho, NULL, 0, NULL),
        BSATTN_ERR_WORKSPACE);
  CHECK(bsattn_fwd_threshold(h, h, h, NULL, 1, 1, 256, 64, 0.5f, 0, 1, 1, NULL, ho, NULL, 0, NULL),
        BSATTN_ERR_NULL);

  /* decode forms */
  CHECK(bsattn_decode_gqa(h, h, h, ci, NULL, 8, 32, 8, 128, 128, 64, 100, 4, ho, ws, 1 << 30, NULL),
        BSATTN_ERR_NULL);
  CHECK(bsattn_decode_gqa(h, h, h, ci, ci, 8, 30, 8, 128, 128, 64, 100, 4, ho, ws, 1 << 30, NULL),
        BSATTN_ERR_SHAPE);
  CHECK(bsattn_decode_gqa(h, h, h, ci, ci, 8, 32, 8, 96, 128, 64, 100, 4, ho, ws, 1 << 30, NULL),
        BSATTN_ERR_UNSUPPORTED);
  CHECK(bsattn_decode_gqa(h, h, h, ci, ci, 8, 32, 8, 128, 128, 64, 100, 4, ho, ws, 16, NULL),
        BSATTN_ERR_WORKSPACE);
  CHECK(bsattn_decode_gqa(h, h, h, ci, ci, big, big, 1, 128, 128, 64, 100, 4, ho, ws, 1 << 30, NULL),
        BSATTN_ERR_UNSUPPORTED);   /* group of 2^31 - 1 heads */
  CHECK(bsattn_decode_gqa(h, h, h, ci, ci, big, 32, 8, 128, 128, 64, 100, 4, ho, ws, (size_t)1 << 62,
                          NULL), BSATTN_ERR_SHAPE);   /* 2^31 - 1 sequences */
  CHECK(bsattn_decode_gqa_noalloc(h, h, h, ci, ci, 64, 64, 4, 128, 128, 64, 100, 64, ho, NULL),
        BSATTN_ERR_WORKSPACE);
  CHECK(bsattn_decode_gqa_mask(h, h, h, ci, NULL, 8, 32, 8, 128, 128, 64, 100, 4, ho, ws, 1 << 30,
                               NULL), BSATTN_ERR_NULL);
  CHECK(bsattn_decode_gqa_paged(h, h, h, ci, ci, NULL, 8, 32, 8, 128, 128, 100, 256, 16, 64, 4, ho,
                                ws, 1 << 30, NULL), BSATTN_ERR_NULL);

  /* sizes whose products would wrap are refused, never wrapped into a small workspace */
  CHECK(bsattn_decode_workspace_bytes(65535, 1 << 22, 128, big) == 0, 1);
  CHECK(bsattn_decode_gqa(h, h, h, ci, ci, 65535, 64, 1, 128, 128, big, 100, big, ho, ws, 1 << 20,
                          NULL), BSATTN_ERR_SHAPE);
  CHECK(bsattn_decode_gqa_noalloc(h, h, h, ci, ci, 65535, 64, 1, 128, 128, big, 100, big, ho, NULL),
        BSATTN_ERR_SHAPE);
  CHECK(bsattn_xattn_workspace_bytes(1, 1, 64, 64 * 100000, 8) == 0, 1);

  /* estimator */
  CHECK(bsattn_xattn_block_sums(NULL, h, 1, 1, 256, 256, 64, 8, 1.0f, 1, fo, ws, 1 << 30, NULL),
        BSATTN_ERR_NULL);
  CHECK(bsattn_xattn_block_sums(h, h, 1, 1, 100, 100, 64, 8, 1.0f, 1, fo, ws, 1 << 30, NULL),
        BSATTN_ERR_SHAPE);
  CHECK(bsattn_build_mask_cumulative(NULL, 1, 1, 4, 4, 0.9f, 1, 1, 1, m, NULL), BSATTN_ERR_NULL);
  CHECK(bsattn_xattn_estimate(h, h, 1, 1, 256, 256, 64, 8, 1.0f, 0.9f, 1, 1, 1, NULL, m, NULL, 0,
                              NULL), BSATTN_ERR_WORKSPACE);

  /* host-only arithmetic over small, large and overflowing arguments */
  const int vals[] = {-1, 0, 1, 2, 7, 64, 65, 1000, 8192, 8193, 65536, 1 << 20, big};
  const int nv = (int)(sizeof(vals) / sizeof(vals[0]));
  size_t acc = 0;
  for (int a = 0; a < nv; ++a)
    for (int b = 0; b < nv; ++b)
      for (int c = 0; c < nv; ++c) {
        acc += bsattn_fwd_workspace_bytes(vals[a], vals[b], vals[c], 64);
        acc += bsattn_fwd_workspace_bytes(vals[a], vals[b], vals[c], 128);
        acc += bsattn_decode_workspace_bytes(vals[a], vals[b], 128, vals[c]);
        acc += bsattn_xattn_workspace_bytes(vals[a], vals[b], vals[c], vals[c], 8);
        acc += bsattn_xattn_workspace_bytes(1, vals[a], vals[b], vals[c], 16);
      }
  acc += bsattn_decode_noalloc_scratch_bytes();
  long long splits = 0;
  for (int B = 1; B <= 64; B *= 2)
    for (int hkv = 1; hkv <= 16; hkv *= 2)
      for (int g = 1; g <= 64; g *= 2)
        for (int sel = 1; sel <= 4096; sel *= 4)
          for (int cus = 1; cus <= 512; cus *= 8) {
            splits += bsattn_decode_num_splits(B, hkv * g, hkv, sel, 128, cus);
            splits += bsattn_decode_num_splits(B, hkv * g, hkv, sel, 64, cus);
          }
  for (int a = 0; a < nv; ++a)
    for (int b = 0; b < nv; ++b) splits += bsattn_decode_num_splits(vals[a], vals[b], 1, vals[a], 128, vals[b]);
  printf("%zu %lld %d\n", acc, splits, bad);
  return bad ? 1 : 0;
}
"""


def _build_dir():
    return os.path.join(os.path.dirname(bsa.LIB_PATH), "_build")


@pytest.mark.skipif(shutil.which("hipcc") is None or not os.path.exists(CLANG),
                    reason="needs hipcc and the ROCm clang")
def test_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    objdir = _build_dir()
    others = [os.path.join(objdir, s.replace(".hip", ".o")) for s in bld.SOURCES if s != "api.hip"]
    if not all(os.path.exists(o) for o in others):
        pytest.skip("library objects not built (run __graft_entry__.build())")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    api_o = tmp_path / "api_san.o"
    r = subprocess.run(["hipcc", *bld.FLAGS, *san, "-g", "-c", os.path.join(bld.CSRC, "api.hip"),
                        "-o", str(api_o)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    lib = tmp_path / "libbsattn_san.so"
    r = subprocess.run(["hipcc", f"--offload-arch={bld.ARCH}", "-shared", "-fPIC", str(api_o), *others,
                        "-o", str(lib)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    src = tmp_path / "harness.c"
    src.write_text(HARNESS)
    exe = tmp_path / "harness"
    r = subprocess.run([CLANG, "-std=c99", "-g", "-fsanitize=address,undefined",
                        "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"), str(src),
                        "-o", str(exe), f"-L{tmp_path}", "-l:libbsattn_san.so",
                        f"-Wl,-rpath,{tmp_path}"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ)
    # leaks: the HIP runtime's own start-up allocations are not this library's
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-3000:]
    assert r.stdout.split()[-1] == "0", r.stdout
