// Internal launchers: host functions that enqueue the kernels.  Arguments are
// validated by the C-ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace bsattn {

// Host side: the largest value a kernel attribute has been raised to on each
// device, so a launcher sets it only when a call needs more than any earlier
// call did (devices 0..63; on others it is set on every call).  Instances
// must have static storage duration (zero-initialised).  Concurrent first
// calls may both set the attribute, which is harmless.
struct DeviceHighWater {
  std::atomic<int> level[64];
  template <class F>
  hipError_t raise_to(int v, F&& set) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const bool cached = dev >= 0 && dev < 64;
    if (cached && level[dev].load(std::memory_order_acquire) >= v) return hipSuccess;
    e = set(v);
    if (e == hipSuccess && cached) {
      int cur = level[dev].load(std::memory_order_relaxed);
      while (cur < v && !level[dev].compare_exchange_weak(cur, v, std::memory_order_acq_rel)) {
      }
    }
    return e;
  }
};

hipError_t launch_mask_topk(const float* scores, int B, int H, int nb, int topk, int dense2,
                            int diag, uint8_t* mask, hipStream_t stream);
hipError_t launch_mask_threshold(const float* scores, int B, int H, int nb, float thr,
                                 int dense2, int diag, uint8_t* mask, hipStream_t stream);
hipError_t launch_compact(const uint8_t* mask, int B, int H, int nb, int causal, int32_t* idx,
                          int32_t* cnt, hipStream_t stream);

// Where a forward work item gets its block list from.
enum PrefillSource {
  kSrcMask = 0,       // mask [B,H,nbq,nbk]
  kSrcList = 1,       // idx [B,H,nbq,nbk] + cnt [B,H,nbq]
  kSrcTopk = 2,       // block scores [B,H,nb,nb]: top-k row selection in the prologue
  kSrcThreshold = 3,  // block scores [B,H,nb,nb]: score > threshold in the prologue
};

struct PrefillArgs {
  const uint16_t* q;     // [B,H,Sq,D]
  const uint16_t* k;     // [B,H,Sk,D]
  const uint16_t* v;     // [B,H,Sk,D]
  uint16_t* out;         // [B,H,Sq,D]
  const uint8_t* mask;   // kSrcMask
  const int32_t* idx;    // kSrcList
  const int32_t* cnt;    // kSrcList
  const float* scores;   // kSrcTopk / kSrcThreshold (square: Sq = Sk)
  uint8_t* mask_out;     // kSrcTopk / kSrcThreshold: the built mask, or nullptr
  int topk;
  float threshold;
  int dense2, diag;      // dense last two rows; force the diagonal
  int src;               // PrefillSource
  int B, H, Sq, Sk, D, nbq, nbk;   // Sq <= Sk: the queries are the last Sq positions
  int causal;
  int ks;                // D = 64: key splits per work item, 1 or 2 (D = 128 always uses 2)
  // Long causal rows split in two (mask-row and block-score sources, square
  // only; split_min = 0: off).
  // Query blocks i >= split_row0 can hold more than split_min key blocks; one
  // extra work-group per such query block takes the second half of its list
  // when it does, both halves leave fp32 partial rows in the workspace, and a
  // merge launch writes those rows' output.  Slot s = bh * (nbq - split_row0)
  // + (i - split_row0) of part_o [slots][2][64][D], part_ml [slots][2][64]
  // (row max, row sum) and part_flag [slots] (1 when the row was split).
  int split_min, split_row0;
  float* part_o;
  float2* part_ml;
  int* part_flag;
};
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);
// Key blocks a causal row must exceed before bsattn_fwd splits it.
constexpr int kSplitMinBlocks = 128;
// Workspace of bsattn_fwd for the long-row split: zero when no causal row of
// an nb-block square problem can exceed kSplitMinBlocks, or when the split
// would need more than kSplitMaxBytes.
constexpr size_t kSplitMaxBytes = size_t(2) << 30;
struct SplitLayout {
  int64_t slots;
  size_t o_off, ml_off, flag_off, bytes;
};
inline SplitLayout split_layout(int B, int H, int nb, int D) {
  SplitLayout L{};
  if (nb <= kSplitMinBlocks) return L;
  const auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  L.slots = (int64_t)B * H * (nb - kSplitMinBlocks);
  L.o_off = 0;
  L.ml_off = up((size_t)L.slots * 2 * 64 * D * sizeof(float));
  L.flag_off = L.ml_off + up((size_t)L.slots * 2 * 64 * sizeof(float2));
  L.bytes = L.flag_off + up((size_t)L.slots * sizeof(int));
  if (L.bytes > kSplitMaxBytes) L = SplitLayout{};
  return L;
}
// LDS one forward work-group needs (K/V ring plus a block list of nbk entries).
size_t prefill_lds_bytes(int D, int nbk);
constexpr size_t kMaxLdsBytes = 160 * 1024;

// How a decode call names its keys.
enum DecodeMode {
  kDecodeIndices = 0,  // packed KV + cu_seqlens, block_indices [B, Hkv, max_sel]
  kDecodeMask = 1,     // packed KV + cu_seqlens, block_mask [B, Hkv, max_sel] (slot j = block j)
  kDecodePaged = 2,    // paged KV + cache_seqlens + block_table, block_indices
};

struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* k;               // packed [total_k, Hkv, D] or paged [num_pages, page_size, Hkv, D]
  const uint16_t* v;               // as k, with Dv in place of D
  const int32_t* cu_seqlens;       // packed modes
  const int32_t* block_indices;    // index and paged modes
  const uint8_t* block_mask;       // mask mode
  const int32_t* cache_seqlens;    // paged mode
  const int32_t* block_table;      // paged mode: [B, max_blocks_per_seq]
  uint16_t* out;   // [B, Hq, Dv]
  float* o_part;   // [B, Hq, ns, Dv]
  float* lse;      // [B, Hq, ns]
  int B, Hq, Hkv, D, Dv, max_sel, total_k, num_splits;   // D: q/k head dim, Dv: v/out head dim
  int page_size, num_pages, max_blocks_per_seq;
  int mode;
};
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

// XAttention block-importance estimate.
struct XattnArgs {
  const uint16_t* q;    // [B,H,Sq,D]
  const uint16_t* k;    // [B,H,Sk,D]
  float* lse;           // workspace [B*H, Sq/stride, nbk]: per (reshaped row, key block) log2-sum-exp2
  float* block_sums;    // [B,H,nbq,nbk]
  float scale_log2;     // log2(e) / (sqrt(D) * stride * norm)
  int BH, Sq, Sk, D, stride, nbq, nbk;
  int causal;
  int ntc, nrt;         // set by the launcher: 128-wide reshaped column / row tiles
};
hipError_t launch_xattn_block_sums(XattnArgs a, hipStream_t stream);
hipError_t launch_mask_cumulative(const float* sums, int B, int H, int nbq, int nbk, float threshold,
                                  int keep_sink, int keep_diag, int causal, uint8_t* mask,
                                  hipStream_t stream);
size_t xattn_lse_bytes(int B, int H, int Sq, int Sk, int stride);
int xattn_max_key_blocks();

}  // namespace bsattn
