// C ABI of the block-sparse attention library: argument checks and launches.
// All checks run before anything is enqueued; see include/bsattn.h.
#include <atomic>
#include <cstring>
#include <math.h>

#include "../../include/bsattn.h"
#include "launch.hpp"

using namespace bsattn;

namespace {

inline hipStream_t as_hip(bsattn_stream_t s) { return reinterpret_cast<hipStream_t>(s); }

inline bool head_dim_ok(int D) { return D == 64 || D == 128; }

// 64-token blocks covering n tokens (0 for n <= 0; no overflow near INT_MAX)
inline int nblocks(int n) {
  return n <= 0 ? 0 : (int)(((long long)n + BSATTN_BLOCK - 1) / BSATTN_BLOCK);
}

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// int32 sizes whose products index 64-bit element offsets
inline bool fits_elems(long double n) { return n < 9.0e18L; }
// a * b * c of sizes that are each an int, without integer overflow (the
// product of three ints can pass 2^63; only its comparison with a bound is
// used, which the 64-bit mantissa keeps exact at these bounds).
inline long double prod3(long long a, long long b, long long c) { return (long double)a * b * c; }

// Split count of the guide's heuristic (TileLang block-sparse Flash-Attention
// guide, §6.3), written for decode: one (batch, KV head) pair is one m-block.
int heuristic_splits(int B, int Hq, int Hkv, int max_sel, int D, int num_cus) {
  const int group = Hq / Hkv;
  const int valid_block_h = group < 64 ? group : 64;
  const long long total_mblocks = (long long)B * (Hq / valid_block_h);
  const long long num_n_blocks = max_sel;
  const long long num_m_blocks = 1;
  const double size_one_kv_head = (double)max_sel * BSATTN_BLOCK * (D + D) * 2.0;
  const double l2 = 50.0 * 1024 * 1024;
  const bool causal_or_local = true;
  const int max_splits = 128;
  if (total_mblocks >= 0.8 * num_cus) {
    if (size_one_kv_head > l2 && num_m_blocks >= 2LL * num_cus && !causal_or_local) {
      long long s = (long long)ceil(size_one_kv_head / l2);
      return (int)(s < max_splits ? s : max_splits);
    }
    return 1;
  }
  if (num_n_blocks <= 4) return 1;
  long long cap = max_splits;
  if (num_cus < cap) cap = num_cus;
  if (num_n_blocks < cap) cap = num_n_blocks;
  double best = 0.0;
  for (long long s = 1; s <= cap; ++s) {
    const double waves = (double)total_mblocks * s / num_cus;
    const double eff = waves / ceil(waves);
    if (eff > best) best = eff;
  }
  for (long long s = 1; s <= cap; ++s) {
    const double waves = (double)total_mblocks * s / num_cus;
    const double eff = waves / ceil(waves);
    if (eff >= 0.85 * best) return (int)s;
  }
  return 1;
}

std::atomic<int> g_cu_count[64];

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    int c = g_cu_count[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (dev < 64 && cus > 0) g_cu_count[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// A decode call's partial outputs (one per batch, query head and split):
// at most 2^31 - 1, so the sizes below cannot wrap.
inline bool decode_parts_ok(int B, int Hq, int ns) { return prod3(B, Hq, ns) <= 2147483647.0L; }

size_t decode_ws(int B, int Hq, int D, int ns) {   // callers check decode_parts_ok first
  if (ns <= 1) return 0;
  const size_t parts = (size_t)B * Hq * ns;
  return align_up(parts * D * sizeof(float)) + align_up(parts * sizeof(float));
}

constexpr size_t kNoAllocScratchBytes = size_t(8) << 20;

// Query heads per KV head the decode takes (the guide's §6.1 block_H = 64).
constexpr int kMaxDecodeGroup = 64;

}  // namespace

// Scratch of the decode entry point that allocates nothing: the split
// stage's partials live in this file-scope device array (one copy per GPU,
// held until the process ends).  In host code `decode_scratch` names a
// host-side stand-in, never the device memory; the device address comes from
// hipGetSymbolAddress, looked up once per device with that device current.
static __device__ __align__(256) unsigned char decode_scratch[kNoAllocScratchBytes];

namespace {

std::atomic<void*> g_decode_scratch[64];

// The device address of decode_scratch on the current device, or nullptr if
// the runtime cannot give it.
void* decode_scratch_ptr() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return nullptr;
  if (dev < 64) {
    void* p = g_decode_scratch[dev].load(std::memory_order_acquire);
    if (p) return p;
  }
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(decode_scratch)) != hipSuccess) return nullptr;
  if (dev < 64 && p) g_decode_scratch[dev].store(p, std::memory_order_release);
  return p;
}

}  // namespace

extern "C" {

const char* bsattn_status_string(bsattn_status s) {
  // A C caller may pass any int: read the code's bits, not the enum value
  // (an out-of-range value of the enum type is undefined in C++).
  int code;
  std::memcpy(&code, &s, sizeof code);
  switch (code) {
    case BSATTN_OK: return "ok";
    case BSATTN_ERR_NULL: return "null pointer argument";
    case BSATTN_ERR_SHAPE: return "size out of range or inconsistent";
    case BSATTN_ERR_UNSUPPORTED: return "unsupported configuration (head dims must be 64 or 128; decode group size <= 64)";
    case BSATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case BSATTN_ERR_HIP: return "HIP runtime error at launch";
  }
  return "unknown status";
}

const char* bsattn_version(void) { return "0.1.0"; }

bsattn_status bsattn_build_mask_topk(const float* scores, int B, int H, int nb, int topk,
                                     int dense_last_two_rows, int force_diagonal, uint8_t* mask,
                                     bsattn_stream_t stream) {
  if (!scores || !mask) return BSATTN_ERR_NULL;
  if (B <= 0 || H <= 0 || nb <= 0 || topk < 0 || topk > nb) return BSATTN_ERR_SHAPE;
  if (prod3(B, H, nb) > 0x7fffffffLL) return BSATTN_ERR_SHAPE;
  return launch_mask_topk(scores, B, H, nb, topk, dense_last_two_rows ? 1 : 0,
                          force_diagonal ? 1 : 0, mask, as_hip(stream)) == hipSuccess
             ? BSATTN_OK
             : BSATTN_ERR_HIP;
}

bsattn_status bsattn_build_mask_threshold(const float* scores, int B, int H, int nb,
                                          float threshold, int dense_last_two_rows,
                                          int force_diagonal, uint8_t* mask,
                                          bsattn_stream_t stream) {
  if (!scores || !mask) return BSATTN_ERR_NULL;
  if (B <= 0 || H <= 0 || nb <= 0) return BSATTN_ERR_SHAPE;
  if (prod3(B, H, nb) > 0x7fffffffLL) return BSATTN_ERR_SHAPE;
  return launch_mask_threshold(scores, B, H, nb, threshold, dense_last_two_rows ? 1 : 0,
                               force_diagonal ? 1 : 0, mask, as_hip(stream)) == hipSuccess
             ? BSATTN_OK
             : BSATTN_ERR_HIP;
}

bsattn_status bsattn_mask_to_indices(const uint8_t* mask, int B, int H, int nb, int is_causal,
                                     int32_t* idx, int32_t* cnt, bsattn_stream_t stream) {
  if (!mask || !idx || !cnt) return BSATTN_ERR_NULL;
  if (B <= 0 || H <= 0 || nb <= 0) return BSATTN_ERR_SHAPE;
  if (prod3(B, H, nb) / 4 + 1 > 0x7fffffffLL) return BSATTN_ERR_SHAPE;
  return launch_compact(mask, B, H, nb, is_causal ? 1 : 0, idx, cnt, as_hip(stream)) == hipSuccess
             ? BSATTN_OK
             : BSATTN_ERR_HIP;
}

size_t bsattn_fwd_workspace_bytes(int B, int H, int S, int D) {
  if (B <= 0 || H <= 0 || S <= 0 || !head_dim_ok(D)) return 0;
  if (prod3(B, H, nblocks(S)) > 0x7fffffffLL) return 0;
  return split_layout(B, H, nblocks(S), D).bytes;
}

// Block lists are held as 16-bit entries in LDS next to the K/V ring.
static bool fwd_key_blocks_ok(int D, int nbk) {
  return nbk <= 65535 && prefill_lds_bytes(D, nbk) <= kMaxLdsBytes;
}

int bsattn_fwd_max_key_blocks(int D) {
  if (!head_dim_ok(D)) return 0;
  int lo = 1, hi = 65535;   // the LDS use grows with nbk: bisect for the last that fits
  if (!fwd_key_blocks_ok(D, lo)) return 0;
  while (lo < hi) {
    const int mid = lo + (hi - lo + 1) / 2;
    if (fwd_key_blocks_ok(D, mid)) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// The shape checks every forward form shares.
static bsattn_status fwd_check(int B, int H, int Sq, int Sk, int D) {
  if (B <= 0 || H <= 0 || Sq <= 0 || Sk < Sq) return BSATTN_ERR_SHAPE;
  if (!head_dim_ok(D)) return BSATTN_ERR_UNSUPPORTED;
  if (prod3(B, H, nblocks(Sq)) > 0x7fffffffLL) return BSATTN_ERR_SHAPE;
  if (!fwd_key_blocks_ok(D, nblocks(Sk))) return BSATTN_ERR_UNSUPPORTED;
  if (!fits_elems((long double)B * H * Sk * D)) return BSATTN_ERR_SHAPE;
  return BSATTN_OK;
}

// Shared checks and launch of the forward forms; `a` carries the
// source-specific pointers (mask, list, or block scores).
static bsattn_status fwd_common(PrefillArgs a, int B, int H, int Sq, int Sk, int D, int is_causal,
                                hipStream_t stream) {
  const bsattn_status st = fwd_check(B, H, Sq, Sk, D);
  if (st != BSATTN_OK) return st;
  a.B = B; a.H = H; a.Sq = Sq; a.Sk = Sk; a.D = D;
  a.nbq = nblocks(Sq); a.nbk = nblocks(Sk);
  a.causal = is_causal ? 1 : 0;
  // D = 64: four waves per item when the items are no more than one round of
  // resident work-groups (four per CU), two otherwise
  const long long items = (long long)B * H * a.nbq;
  a.ks = (D == 64 && items <= 4LL * device_cu_count()) ? 2 : 1;
  return launch_prefill(a, stream) == hipSuccess ? BSATTN_OK : BSATTN_ERR_HIP;
}

static PrefillArgs fwd_args(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* out,
                            int src) {
  PrefillArgs a{};
  a.q = q; a.k = k; a.v = v; a.out = out;
  a.src = src;
  return a;
}

// The long-row split of a causal square forward: checks the workspace and
// points the split fields of `a` into it (nothing to do when no row can
// exceed the split threshold).
static bsattn_status set_long_row_split(PrefillArgs& a, int B, int H, int S, int D, int is_causal,
                                        void* workspace, size_t workspace_bytes) {
  if (B <= 0 || H <= 0 || S <= 0 || !head_dim_ok(D)) return BSATTN_OK;   // fwd_common reports it
  const size_t need = bsattn_fwd_workspace_bytes(B, H, S, D);
  if (need == 0 || !is_causal) return BSATTN_OK;
  if (!workspace || workspace_bytes < need || (uintptr_t)workspace % 16 != 0)
    return BSATTN_ERR_WORKSPACE;
  const SplitLayout L = split_layout(B, H, nblocks(S), D);
  unsigned char* ws = (unsigned char*)workspace;
  a.split_min = kSplitMinBlocks;
  a.split_row0 = kSplitMinBlocks;   // causal row i holds at most i + 1 blocks
  a.part_o = (float*)(ws + L.o_off);
  a.part_ml = (float2*)(ws + L.ml_off);
  a.part_flag = (int*)(ws + L.flag_off);
  return BSATTN_OK;
}

bsattn_status bsattn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         const uint8_t* block_mask, int B, int H, int S, int D, int is_causal,
                         uint16_t* out, void* workspace, size_t workspace_bytes,
                         bsattn_stream_t stream) {
  if (!q || !k || !v || !block_mask || !out) return BSATTN_ERR_NULL;
  PrefillArgs a = fwd_args(q, k, v, out, kSrcMask);
  a.mask = block_mask;
  const bsattn_status st = set_long_row_split(a, B, H, S, D, is_causal, workspace, workspace_bytes);
  if (st != BSATTN_OK) return st;
  return fwd_common(a, B, H, S, S, D, is_causal, as_hip(stream));
}

bsattn_status bsattn_fwd_chunk(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                               const uint8_t* block_mask, int B, int H, int Sq, int Sk, int D,
                               int is_causal, uint16_t* out, bsattn_stream_t stream) {
  if (!q || !k || !v || !block_mask || !out) return BSATTN_ERR_NULL;
  PrefillArgs a = fwd_args(q, k, v, out, kSrcMask);
  a.mask = block_mask;
  return fwd_common(a, B, H, Sq, Sk, D, is_causal, as_hip(stream));
}

bsattn_status bsattn_fwd_indices(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                 const int32_t* idx, const int32_t* cnt, int B, int H, int S,
                                 int D, int is_causal, uint16_t* out, bsattn_stream_t stream) {
  if (!q || !k || !v || !idx || !cnt || !out) return BSATTN_ERR_NULL;
  PrefillArgs a = fwd_args(q, k, v, out, kSrcList);
  a.idx = idx; a.cnt = cnt;
  return fwd_common(a, B, H, S, S, D, is_causal, as_hip(stream));
}

// The fused forms hold a row's order keys in registers, 4 per lane.
static bool fused_nb_ok(int D, int S) {
  (void)D;
  return nblocks(S) <= 256;
}

// Rows too long for the one-launch form: the builder writes the mask to
// mask_out, then the mask-row forward runs on it (the same mask bytes and
// the same output as one launch would give).  Every check runs before the
// first launch.
extern "C++" template <class Build>
static bsattn_status fused_two_launch(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                      int B, int H, int S, int D, int is_causal, uint8_t* mask_out,
                                      uint16_t* out, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream, Build build) {
  if (!mask_out) return BSATTN_ERR_UNSUPPORTED;
  PrefillArgs a = fwd_args(q, k, v, out, kSrcMask);
  a.mask = mask_out;
  bsattn_status st = set_long_row_split(a, B, H, S, D, is_causal, workspace, workspace_bytes);
  if (st == BSATTN_OK) st = fwd_check(B, H, S, S, D);
  if (st != BSATTN_OK) return st;
  if (build() != hipSuccess) return BSATTN_ERR_HIP;
  return fwd_common(a, B, H, S, S, D, is_causal, stream);
}

bsattn_status bsattn_fwd_topk(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              const float* block_scores, int B, int H, int S, int D, int topk,
                              int dense_last_two_rows, int force_diagonal, int is_causal,
                              uint8_t* mask_out, uint16_t* out, void* workspace,
                              size_t workspace_bytes, bsattn_stream_t stream) {
  if (!q || !k || !v || !block_scores || !out) return BSATTN_ERR_NULL;
  if (S > 0 && (topk < 0 || topk > nblocks(S))) return BSATTN_ERR_SHAPE;
  if (S > 0 && head_dim_ok(D) && !fused_nb_ok(D, S))
    return fused_two_launch(q, k, v, B, H, S, D, is_causal, mask_out, out, workspace,
                            workspace_bytes, as_hip(stream), [&]() {
                              return launch_mask_topk(block_scores, B, H, nblocks(S), topk,
                                                      dense_last_two_rows ? 1 : 0,
                                                      force_diagonal ? 1 : 0, mask_out,
                                                      as_hip(stream));
                            });
  PrefillArgs a = fwd_args(q, k, v, out, kSrcTopk);
  a.scores = block_scores; a.mask_out = mask_out; a.topk = topk;
  a.dense2 = dense_last_two_rows ? 1 : 0; a.diag = force_diagonal ? 1 : 0;
  const bsattn_status st = set_long_row_split(a, B, H, S, D, is_causal, workspace, workspace_bytes);
  if (st != BSATTN_OK) return st;
  return fwd_common(a, B, H, S, S, D, is_causal, as_hip(stream));
}

bsattn_status bsattn_fwd_threshold(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                   const float* block_scores, int B, int H, int S, int D,
                                   float threshold, int dense_last_two_rows, int force_diagonal,
                                   int is_causal, uint8_t* mask_out, uint16_t* out,
                                   void* workspace, size_t workspace_bytes,
                                   bsattn_stream_t stream) {
  if (!q || !k || !v || !block_scores || !out) return BSATTN_ERR_NULL;
  if (S > 0 && head_dim_ok(D) && !fused_nb_ok(D, S))
    return fused_two_launch(q, k, v, B, H, S, D, is_causal, mask_out, out, workspace,
                            workspace_bytes, as_hip(stream), [&]() {
                              return launch_mask_threshold(block_scores, B, H, nblocks(S),
                                                           threshold, dense_last_two_rows ? 1 : 0,
                                                           force_diagonal ? 1 : 0, mask_out,
                                                           as_hip(stream));
                            });
  PrefillArgs a = fwd_args(q, k, v, out, kSrcThreshold);
  a.scores = block_scores; a.mask_out = mask_out; a.threshold = threshold;
  a.dense2 = dense_last_two_rows ? 1 : 0; a.diag = force_diagonal ? 1 : 0;
  const bsattn_status st = set_long_row_split(a, B, H, S, D, is_causal, workspace, workspace_bytes);
  if (st != BSATTN_OK) return st;
  return fwd_common(a, B, H, S, S, D, is_causal, as_hip(stream));
}

int bsattn_decode_num_splits(int B, int Hq, int Hkv, int max_selected_blocks, int D,
                             int num_cus) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || max_selected_blocks <= 0 || D <= 0 ||
      num_cus <= 0)
    return 0;
  return heuristic_splits(B, Hq, Hkv, max_selected_blocks, D, num_cus);
}

int bsattn_decode_default_splits(int B, int Hq, int Hkv, int max_selected_blocks, int D) {
  const int cus = device_cu_count();
  if (cus <= 0) return 0;
  int s = bsattn_decode_num_splits(B, Hq, Hkv, max_selected_blocks, D, cus);
  if (s > max_selected_blocks) s = max_selected_blocks;
  return s;
}

size_t bsattn_decode_workspace_bytes(int B, int Hq, int D, int num_splits) {
  if (B <= 0 || Hq <= 0 || D <= 0 || num_splits <= 0) return 0;
  if (D > 65536 || !decode_parts_ok(B, Hq, num_splits)) return 0;
  return decode_ws(B, Hq, D, num_splits);
}

}  // extern "C"

namespace {

// Shared checks and launch of the three decode forms; `a` carries the
// form-specific pointers and sizes, `slots` is the per-(batch, KV head) slot
// count the splits divide (max_selected_blocks, or num_blocks of a mask).
bsattn_status decode_common(DecodeArgs a, int slots, int num_splits, void* workspace,
                            size_t workspace_bytes, hipStream_t stream,
                            bool static_scratch = false) {
  if (!a.q || !a.k || !a.v || !a.out) return BSATTN_ERR_NULL;
  if (a.B <= 0 || a.Hq <= 0 || a.Hkv <= 0 || slots <= 0) return BSATTN_ERR_SHAPE;
  if (a.Hq % a.Hkv != 0) return BSATTN_ERR_SHAPE;
  if (num_splits > slots) return BSATTN_ERR_SHAPE;
  if (!head_dim_ok(a.D) || !head_dim_ok(a.Dv) || a.Hq / a.Hkv > kMaxDecodeGroup)
    return BSATTN_ERR_UNSUPPORTED;
  // grid: splits x (KV heads x 16-head column tiles) x batch
  if (a.B > 65535 || (long long)a.Hkv * ((a.Hq / a.Hkv + 15) / 16) > 65535) return BSATTN_ERR_SHAPE;
  int ns = num_splits;
  if (ns <= 0) {
    ns = bsattn_decode_default_splits(a.B, a.Hq, a.Hkv, slots, a.D);
    if (ns <= 0) return BSATTN_ERR_HIP;
  }
  if (!decode_parts_ok(a.B, a.Hq, ns)) return BSATTN_ERR_SHAPE;
  const size_t need = decode_ws(a.B, a.Hq, a.Dv, ns);
  if (static_scratch && need > 0) {
    // the no-allocation form: the partials go to the static scratch array
    if (need > kNoAllocScratchBytes) return BSATTN_ERR_WORKSPACE;
    workspace = decode_scratch_ptr();
    if (!workspace) return BSATTN_ERR_HIP;
    workspace_bytes = kNoAllocScratchBytes;
  }
  if (need > 0 && (!workspace || workspace_bytes < need)) return BSATTN_ERR_WORKSPACE;
  const size_t parts = (size_t)a.B * a.Hq * ns;
  a.o_part = (float*)workspace;
  a.lse = need ? (float*)((char*)workspace + align_up(parts * a.Dv * sizeof(float))) : nullptr;
  a.max_sel = slots;
  a.num_splits = ns;
  return launch_decode(a, stream) == hipSuccess ? BSATTN_OK : BSATTN_ERR_HIP;
}

}  // namespace

extern "C" {

bsattn_status bsattn_decode_gqa(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                const int32_t* cu_seqlens_k, const int32_t* block_indices, int B,
                                int Hq, int Hkv, int D, int Dv, int max_selected_blocks, int total_k,
                                int num_splits, uint16_t* out, void* workspace,
                                size_t workspace_bytes, bsattn_stream_t stream) {
  if (!q || !k || !v || !out || !cu_seqlens_k || !block_indices) return BSATTN_ERR_NULL;
  if (total_k <= 0) return BSATTN_ERR_SHAPE;
  DecodeArgs a{};
  a.q = q; a.k = k; a.v = v; a.out = out;
  a.cu_seqlens = cu_seqlens_k; a.block_indices = block_indices;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.D = D; a.Dv = Dv; a.total_k = total_k;
  a.mode = kDecodeIndices;
  return decode_common(a, max_selected_blocks, num_splits, workspace, workspace_bytes,
                       as_hip(stream));
}

bsattn_status bsattn_decode_gqa_noalloc(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                        const int32_t* cu_seqlens_k, const int32_t* block_indices,
                                        int B, int Hq, int Hkv, int D, int Dv, int max_selected_blocks,
                                        int total_k, int num_splits, uint16_t* out,
                                        bsattn_stream_t stream) {
  if (!q || !k || !v || !out || !cu_seqlens_k || !block_indices) return BSATTN_ERR_NULL;
  if (total_k <= 0) return BSATTN_ERR_SHAPE;
  DecodeArgs a{};
  a.q = q; a.k = k; a.v = v; a.out = out;
  a.cu_seqlens = cu_seqlens_k; a.block_indices = block_indices;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.D = D; a.Dv = Dv; a.total_k = total_k;
  a.mode = kDecodeIndices;
  return decode_common(a, max_selected_blocks, num_splits, nullptr, 0, as_hip(stream), true);
}

size_t bsattn_decode_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

bsattn_status bsattn_decode_gqa_mask(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                     const int32_t* cu_seqlens_k, const uint8_t* block_mask, int B,
                                     int Hq, int Hkv, int D, int Dv, int num_blocks, int total_k,
                                     int num_splits, uint16_t* out, void* workspace,
                                     size_t workspace_bytes, bsattn_stream_t stream) {
  if (!q || !k || !v || !out || !cu_seqlens_k || !block_mask) return BSATTN_ERR_NULL;
  if (total_k <= 0) return BSATTN_ERR_SHAPE;
  DecodeArgs a{};
  a.q = q; a.k = k; a.v = v; a.out = out;
  a.cu_seqlens = cu_seqlens_k; a.block_mask = block_mask;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.D = D; a.Dv = Dv; a.total_k = total_k;
  a.mode = kDecodeMask;
  return decode_common(a, num_blocks, num_splits, workspace, workspace_bytes, as_hip(stream));
}

bsattn_status bsattn_decode_gqa_paged(const uint16_t* q, const uint16_t* k_cache,
                                      const uint16_t* v_cache, const int32_t* cache_seqlens,
                                      const int32_t* block_table, const int32_t* block_indices,
                                      int B, int Hq, int Hkv, int D, int Dv, int num_pages, int page_size,
                                      int max_blocks_per_seq, int max_selected_blocks,
                                      int num_splits, uint16_t* out, void* workspace,
                                      size_t workspace_bytes, bsattn_stream_t stream) {
  if (!q || !k_cache || !v_cache || !out || !cache_seqlens || !block_table || !block_indices)
    return BSATTN_ERR_NULL;
  if (num_pages <= 0 || page_size <= 0 || max_blocks_per_seq <= 0) return BSATTN_ERR_SHAPE;
  if (page_size % BSATTN_BLOCK != 0) return BSATTN_ERR_SHAPE;
  if (!fits_elems((long double)num_pages * page_size * (Hkv > 0 ? Hkv : 1) * 128 * 2))
    return BSATTN_ERR_SHAPE;
  DecodeArgs a{};
  a.q = q; a.k = k_cache; a.v = v_cache; a.out = out;
  a.cache_seqlens = cache_seqlens; a.block_table = block_table; a.block_indices = block_indices;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.D = D; a.Dv = Dv;
  a.num_pages = num_pages; a.page_size = page_size; a.max_blocks_per_seq = max_blocks_per_seq;
  a.mode = kDecodePaged;
  return decode_common(a, max_selected_blocks, num_splits, workspace, workspace_bytes,
                       as_hip(stream));
}

}  // extern "C"

// ---- XAttention block-importance estimator ----

namespace {

bool xattn_shape_ok(int B, int H, int Sq, int Sk, int stride) {
  if (B <= 0 || H <= 0 || Sq <= 0 || Sk < Sq) return false;
  if (stride <= 0 || Sq % stride != 0 || Sk % stride != 0) return false;
  if ((Sk - Sq) % BSATTN_BLOCK != 0) return false;
  return (long long)B * H <= 65535;
}

bool xattn_stride_ok(int stride) { return stride == 4 || stride == 8 || stride == 16; }

size_t xattn_sums_bytes(int B, int H, int Sq, int Sk) {
  return (size_t)B * H * nblocks(Sq) * nblocks(Sk) * sizeof(float);
}

bsattn_status xattn_sums_common(const uint16_t* q, const uint16_t* k, int B, int H, int Sq, int Sk,
                                int D, int stride, float norm, int is_causal, float* block_sums,
                                void* workspace, size_t workspace_bytes, bool sums_in_ws,
                                hipStream_t stream) {
  if (!xattn_shape_ok(B, H, Sq, Sk, stride)) return BSATTN_ERR_SHAPE;
  if (!(norm > 0.0f) || !isfinite(norm)) return BSATTN_ERR_SHAPE;
  if (!head_dim_ok(D) || !xattn_stride_ok(stride)) return BSATTN_ERR_UNSUPPORTED;
  if (nblocks(Sk) > xattn_max_key_blocks()) return BSATTN_ERR_UNSUPPORTED;
  if (!fits_elems((long double)B * H * Sk * D)) return BSATTN_ERR_SHAPE;
  const size_t lse_bytes = align_up(xattn_lse_bytes(B, H, Sq, Sk, stride));
  const size_t need = lse_bytes + align_up(xattn_sums_bytes(B, H, Sq, Sk));
  if (!workspace || workspace_bytes < need) return BSATTN_ERR_WORKSPACE;
  XattnArgs a{};
  a.q = q;
  a.k = k;
  a.lse = (float*)workspace;
  a.block_sums = sums_in_ws ? (float*)((char*)workspace + lse_bytes) : block_sums;
  a.scale_log2 = (float)(1.4426950408889634 / (sqrt((double)D) * stride * (double)norm));
  a.BH = B * H;
  a.Sq = Sq;
  a.Sk = Sk;
  a.D = D;
  a.stride = stride;
  a.nbq = nblocks(Sq);
  a.nbk = nblocks(Sk);
  a.causal = is_causal ? 1 : 0;
  return launch_xattn_block_sums(a, stream) == hipSuccess ? BSATTN_OK : BSATTN_ERR_HIP;
}

bsattn_status cumulative_check(int B, int H, int nbq, int nbk) {
  if (B <= 0 || H <= 0 || nbq <= 0 || nbk < nbq) return BSATTN_ERR_SHAPE;
  if (prod3(B, H, nbq) > 0x7fffffffLL) return BSATTN_ERR_SHAPE;
  if (nbk > xattn_max_key_blocks()) return BSATTN_ERR_UNSUPPORTED;
  return BSATTN_OK;
}

}  // namespace

extern "C" {

size_t bsattn_xattn_workspace_bytes(int B, int H, int Sq, int Sk, int stride) {
  if (!xattn_shape_ok(B, H, Sq, Sk, stride)) return 0;
  if (nblocks(Sk) > xattn_max_key_blocks()) return 0;   // unsupported: no size can serve it
  return align_up(xattn_lse_bytes(B, H, Sq, Sk, stride)) +
         align_up(xattn_sums_bytes(B, H, Sq, Sk));
}

bsattn_status bsattn_xattn_block_sums(const uint16_t* q, const uint16_t* k, int B, int H, int Sq,
                                      int Sk, int D, int stride, float norm, int is_causal,
                                      float* block_sums, void* workspace, size_t workspace_bytes,
                                      bsattn_stream_t stream) {
  if (!q || !k || !block_sums) return BSATTN_ERR_NULL;
  return xattn_sums_common(q, k, B, H, Sq, Sk, D, stride, norm, is_causal, block_sums, workspace,
                           workspace_bytes, false, as_hip(stream));
}

bsattn_status bsattn_build_mask_cumulative(const float* block_sums, int B, int H, int nbq, int nbk,
                                           float threshold, int keep_sink, int keep_diagonal,
                                           int is_causal, uint8_t* mask, bsattn_stream_t stream) {
  if (!block_sums || !mask) return BSATTN_ERR_NULL;
  const bsattn_status st = cumulative_check(B, H, nbq, nbk);
  if (st != BSATTN_OK) return st;
  return launch_mask_cumulative(block_sums, B, H, nbq, nbk, threshold, keep_sink ? 1 : 0,
                                keep_diagonal ? 1 : 0, is_causal ? 1 : 0, mask,
                                as_hip(stream)) == hipSuccess
             ? BSATTN_OK
             : BSATTN_ERR_HIP;
}

bsattn_status bsattn_xattn_estimate(const uint16_t* q, const uint16_t* k, int B, int H, int Sq,
                                    int Sk, int D, int stride, float norm, float threshold,
                                    int keep_sink, int keep_diagonal, int is_causal,
                                    float* block_sums, uint8_t* mask, void* workspace,
                                    size_t workspace_bytes, bsattn_stream_t stream) {
  if (!q || !k || !mask) return BSATTN_ERR_NULL;
  if (xattn_shape_ok(B, H, Sq, Sk, stride)) {
    const bsattn_status st = cumulative_check(B, H, nblocks(Sq), nblocks(Sk));
    if (st != BSATTN_OK) return st;
  }
  const bool in_ws = block_sums == nullptr;
  const bsattn_status st =
      xattn_sums_common(q, k, B, H, Sq, Sk, D, stride, norm, is_causal, block_sums, workspace,
                        workspace_bytes, in_ws, as_hip(stream));
  if (st != BSATTN_OK) return st;
  const float* sums =
      in_ws ? (const float*)((const char*)workspace + align_up(xattn_lse_bytes(B, H, Sq, Sk, stride)))
            : block_sums;
  return launch_mask_cumulative(sums, B, H, nblocks(Sq), nblocks(Sk), threshold, keep_sink ? 1 : 0,
                                keep_diagonal ? 1 : 0, is_causal ? 1 : 0, mask,
                                as_hip(stream)) == hipSuccess
             ? BSATTN_OK
             : BSATTN_ERR_HIP;
}

}  // extern "C"
