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

// One wave per score row: the row's order keys sit in LDS; lane owns columns
// lane, lane+64, ... and counts the keys above each of its own.
__global__ __launch_bounds__(kWaveRows * kWave) void mask_topk_wave_kernel(
    const float* __restrict__ scores, int64_t rows, int nb, int topk, int dense2, int diag,
    uint8_t* __restrict__ mask) {
  __shared__ uint64_t keys[kWaveRows][kWaveMaxNb];
  const int w = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int64_t row = (int64_t)blockIdx.x * kWaveRows + w;
  if (row >= rows) return;  // the whole wave leaves; only wave-level syncs below
  const int i = (int)(row % nb);
  const float* x = scores + row * (int64_t)nb;
  uint8_t* out = mask + row * (int64_t)nb;

  const bool dense_row = dense2 && i >= nb - 2;
  if (dense_row || topk >= nb || topk == 0) {
    const bool all = dense_row || topk >= nb;
    for (int j = lane; j < nb; j += kWave) out[j] = ((j <= i) && (all || (diag && j == i))) ? 1 : 0;
    return;
  }
  uint64_t* kr = keys[w];
  for (int c = lane; c < nb; c += kWave) kr[c] = rank_key(x[c], c);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  for (int j0 = 0; j0 < nb; j0 += kWave) {
    const int j = j0 + lane;
    if (j0 > i) {            // the whole group lies above the diagonal
      if (j < nb) out[j] = 0;
      continue;
    }
    const uint64_t kj = (j < nb) ? kr[j] : ~0ull;
    int beat = 0;
    for (int c = 0; c < nb; ++c) beat += kr[c] > kj;
    if (j < nb) {
      bool pick;
      if (j > i) pick = false;
      else if (diag && j == i) pick = true;
      else pick = beat < topk;
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
    hipLaunchKernelGGL(mask_topk_wave_kernel, dim3((unsigned)blocks), dim3(kWaveRows * kWave), 0,
                       stream, scores, rows, nb, topk, dense2, diag, mask);
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
