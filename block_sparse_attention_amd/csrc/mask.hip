// Block-mask builders and row compaction (gfx950).
//
// Top-k and threshold builders follow the TileLang block-sparse
// Flash-Attention guide, §3.1 and §3.2: select per query-block row, optionally
// make the last two rows dense, cut above the diagonal (causal tril); the
// diagonal block is then forced on as in the XAttention guide ("algorithm
// flow", phase 3).  Compaction turns a mask row into the ascending list of
// selected key blocks, i.e. the guide's §4.4 loop bound and block-skip branch
// as data.
#include "common.hpp"
#include "launch.hpp"

namespace bsattn {

namespace {

constexpr int kTopkThreads = 256;
constexpr int kTopkChunk = 2048;  // floats of the score row staged in LDS at a time

// One work-group per score row.  Column j (j <= i) is selected when fewer
// than topk columns beat it; c beats j when x[c] > x[j], or x[c] == x[j] and
// c < j (ties go to the lower column).  Columns j > i are cut by tril, so
// they are never ranked, but they still take part as competitors.
__global__ __launch_bounds__(kTopkThreads) void mask_topk_kernel(const float* __restrict__ scores,
                                                                 int nb, int topk, int dense2,
                                                                 int diag,
                                                                 uint8_t* __restrict__ mask) {
  __shared__ float xs[kTopkChunk];
  const int64_t row = blockIdx.x;
  const int i = (int)(row % nb);
  const float* x = scores + row * (int64_t)nb;
  uint8_t* out = mask + row * (int64_t)nb;
  const int tid = threadIdx.x;

  const bool dense_row = dense2 && i >= nb - 2;
  if (dense_row || topk >= nb || topk == 0) {
    // Every column up to the diagonal is selected (dense row or topk = nb),
    // or none is (topk = 0) apart from the forced diagonal.
    const bool all = dense_row || topk >= nb;
    for (int j = tid; j < nb; j += kTopkThreads) {
      bool pick = (j <= i) && (all || (diag && j == i));
      out[j] = pick ? 1 : 0;
    }
    return;
  }

  for (int j0 = 0; j0 < nb; j0 += kTopkThreads) {
    const int j = j0 + tid;
    const bool ranked = j < nb && j <= i && !(diag && j == i);
    const float xj = (j < nb) ? x[j] : 0.0f;
    int beat = 0;
    for (int c0 = 0; c0 < nb; c0 += kTopkChunk) {
      const int cn = min(kTopkChunk, nb - c0);
      __syncthreads();
      for (int c = tid; c < cn; c += kTopkThreads) xs[c] = x[c0 + c];
      __syncthreads();
      if (ranked && beat < topk) {
        // columns before j win ties, columns after j must be strictly larger
        const int split = min(max(j - c0, 0), cn);
        for (int c = 0; c < split; ++c) beat += (xs[c] >= xj);
        for (int c = split; c < cn; ++c) beat += (xs[c] > xj) && (c0 + c != j);
      }
    }
    if (j < nb) {
      bool pick;
      if (j > i) pick = false;
      else if (diag && j == i) pick = true;
      else pick = beat < topk;
      out[j] = pick ? 1 : 0;
    }
  }
}


constexpr int kWaveRows = 4;        // rows per work-group, one wave each
constexpr int kWaveMaxNb = 1024;    // rows up to this length use the one-wave kernel

// One wave per score row: the row's order keys sit in registers, lane l
// holding columns l, l+64, ... (NCH chunks of 64), and a radix select over
// the wave (wave_topk_cut) finds the top-k cut.
template <int NCH>
__global__ __launch_bounds__(kWaveRows * kWave) void mask_topk_wave_kernel(
    const float* __restrict__ scores, int64_t rows, int nb, int topk, int dense2, int diag,
    uint8_t* __restrict__ mask) {
  const int w = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int64_t row = (int64_t)blockIdx.x * kWaveRows + w;
  if (row >= rows) return;  // the whole wave leaves; only wave-level operations below
  const int i = (int)(row % nb);
  const float* x = scores + row * (int64_t)nb;
  uint8_t* out = mask + row * (int64_t)nb;
  const int nch = (nb + kWave - 1) / kWave;

  const bool dense_row = dense2 && i >= nb - 2;
  const bool all = dense_row || topk >= nb;
  const bool ranked = !all && topk > 0;
  uint64_t key[NCH];
  uint64_t hm = 0, prefix = 0;
  if (ranked) {
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
      const int c = kWave * u + lane;
      key[u] = c < nb ? rank_key(x[c], c) : 0ull;   // 0 is below every real key
    }
    wave_topk_cut(key, nch, topk, hm, prefix);
  }
#pragma unroll
  for (int u = 0; u < NCH; ++u) {
    const int j = kWave * u + lane;
    if (u < nch && j < nb) {
      bool pick;
      if (j > i) pick = false;                 // tril
      else if (diag && j == i) pick = true;    // forced diagonal
      else if (all) pick = true;
      else pick = ranked && (key[u] & hm) >= prefix;
      out[j] = pick ? 1 : 0;
    }
  }
}

__global__ __launch_bounds__(256) void mask_threshold_kernel(const float* __restrict__ scores,
                                                             int64_t total, int nb, float thr,
                                                             int dense2, int diag,
                                                             uint8_t* __restrict__ mask) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int j = (int)(e % nb);
    const int i = (int)((e / nb) % nb);
    bool pick = scores[e] > thr;
    if (dense2 && i >= nb - 2) pick = true;
    if (j > i) pick = false;
    if (diag && j == i) pick = true;
    mask[e] = pick ? 1 : 0;
  }
}

// One wave per mask row: a 64-column ballot gives each selected column its
// position in the list.
__global__ __launch_bounds__(256) void compact_kernel(const uint8_t* __restrict__ mask,
                                                      int64_t rows, int nb, int causal,
                                                      int32_t* __restrict__ idx,
                                                      int32_t* __restrict__ cnt) {
  const int64_t row = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (row >= rows) return;
  const int lane = threadIdx.x % kWave;
  const int i = (int)(row % nb);
  const uint8_t* m = mask + row * (int64_t)nb;
  int32_t* out = idx + row * (int64_t)nb;
  const int lim = causal ? min(i + 1, nb) : nb;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int running = 0;
  for (int c0 = 0; c0 < lim; c0 += kWave) {
    const int j = c0 + lane;
    const bool sel = j < lim && m[j] != 0;
    const uint64_t bits = wave_ballot(sel);
    if (sel) out[running + __popcll(bits & below)] = j;
    running += __popcll(bits);
  }
  for (int j = running + lane; j < nb; j += kWave) out[j] = -1;
  if (lane == 0) cnt[row] = running;
}

}  // namespace

hipError_t launch_mask_topk(const float* scores, int B, int H, int nb, int topk, int dense2,
                            int diag, uint8_t* mask, hipStream_t stream) {
  const int64_t rows = (int64_t)B * H * nb;
  if (nb <= kWaveMaxNb) {
    const int64_t blocks = (rows + kWaveRows - 1) / kWaveRows;
    const dim3 grid((unsigned)blocks), block(kWaveRows * kWave);
#define BSATTN_TOPK(NCH)                                                                           \
  hipLaunchKernelGGL(mask_topk_wave_kernel<NCH>, grid, block, 0, stream, scores, rows, nb, topk, \
                     dense2, diag, mask)
    if (nb <= 64) BSATTN_TOPK(1);
    else if (nb <= 128) BSATTN_TOPK(2);
    else if (nb <= 256) BSATTN_TOPK(4);
    else if (nb <= 512) BSATTN_TOPK(8);
    else BSATTN_TOPK(16);
#undef BSATTN_TOPK
  } else {
    hipLaunchKernelGGL(mask_topk_kernel, dim3((unsigned)rows), dim3(kTopkThreads), 0, stream,
                       scores, nb, topk, dense2, diag, mask);
  }
  return hipGetLastError();
}

hipError_t launch_mask_threshold(const float* scores, int B, int H, int nb, float thr,
                                 int dense2, int diag, uint8_t* mask, hipStream_t stream) {
  const int64_t total = (int64_t)B * H * nb * nb;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(mask_threshold_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, scores,
                     total, nb, thr, dense2, diag, mask);
  return hipGetLastError();
}

hipError_t launch_compact(const uint8_t* mask, int B, int H, int nb, int causal, int32_t* idx,
                          int32_t* cnt, hipStream_t stream) {
  const int64_t rows = (int64_t)B * H * nb;
  const int64_t blocks = (rows + 3) / 4;
  hipLaunchKernelGGL(compact_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, mask, rows, nb,
                     causal, idx, cnt);
  return hipGetLastError();
}

}  // namespace bsattn
