// XAttention block-importance estimator (gfx950): the block scores upstream
// of the block mask (XAttention guide, "algorithm flow" phases 1-3).
//
// Stride reshape in inverse mode (the guide's stride-reshape section): with
// stride s, reshaped key row t' is key rows t's .. t's+s-1 concatenated, and
// reshaped query row r' is query rows r's+s-1 down to r's.  The reshaped
// logit is therefore
//     L[r', t'] = sum_j q[r's + s-1-j] . k[t's + j]  / (sqrt(D) * s * norm),
// a GEMM with inner dimension s*D.  No reshaped copy is made: K' is K read
// as [Sk/s, s*D] rows (contiguous), and Q' is Q read the same way with the s
// sub-rows of each reshaped row taken in reverse, which is only a different
// source address per 64-dimension chunk of the inner loop (the guide's fused
// reshape-GEMM does the same with pointer arithmetic).
//
// Three kernels:
// * xattn_lse_kernel: one 128 x 128 tile of L^T per work-group (4 waves, each
//   64 x 64 from 32x32x16 bf16 MFMAs; operands stream HBM -> LDS by direct
//   loads, double-buffered over 64-dimension chunks; tiles ordered so the
//   ones resident on an XCD share operand strips in its L2).  The tile's epilogue
//   reduces every (reshaped row, 64-token key block) to the log2-sum-exp2 of
//   its scaled logits and stores it.  Tiles are independent: the row softmax
//   needs the whole row, and per-block log-sums let the next kernel normalise
//   without a second pass over the GEMM.
// * xattn_blocksum_kernel: per (query block, all key blocks): each reshaped
//   row's log-normaliser from its block log-sums, then the block sums of the
//   softmax weights (the guide's softmax + block-sum kernel description).
// * mask_cumulative_kernel: per query-block row, block selection by
//   cumulative weight (the guide's block-selection section): sink and
//   diagonal kept, the rest ranked by weight and kept while the weight
//   ranked above is below threshold * total.  Sums are float64, the total in
//   ascending column order and the ranked sum in rank order, one term at a
//   time; the ranking is a bitonic sort of order keys held in registers.
#include <math.h>

#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace bsattn {

namespace {

// A tile is 64 WT reshaped keys x 128 reshaped queries, computed by 2 WT waves
// of 64 x 64 each.
constexpr int kXTileR = 128;          // reshaped queries (rows of L) per tile
constexpr int kXChunk = 64;           // inner dimensions per LDS stage
template <int WT>
struct XTile {
  static constexpr int kWaves = 2 * WT;
  static constexpr int kThreads = kWaves * kWave;
  static constexpr int kT = 64 * WT;                       // reshaped keys per tile
  static constexpr int kOpBytesK = kT * kXChunk * 2;       // K' part of a stage
  static constexpr int kStageBytes = (kT + kXTileR) * kXChunk * 2;
  static constexpr int kLdsBytes = 2 * kStageBytes;        // two stages
};
template <int WT>
constexpr int kXThreadsFor = 2 * WT * kWave;
#ifndef BSATTN_XBAND
#define BSATTN_XBAND 8
#endif
constexpr int kXBand = BSATTN_XBAND;  // row tiles walked together (L2 reuse)
#ifndef BSATTN_XWT
#define BSATTN_XWT 2
#endif
constexpr int kXWT = BSATTN_XWT;      // waves along the reshaped keys (tile: 64 kXWT keys)

// 16-byte granule g of LDS row r (128 bytes) is stored at granule g ^ xswz(r):
// the 32-row, 16-byte-per-lane operand reads then touch every bank once.
__device__ __forceinline__ int xswz(int r) { return (r >> 1) & 7; }

// One work-group per (head, row tile, column tile).  A tile whose columns all
// lie past the causal limit of every row it holds is not computed.
template <int D, int S, int WT>
__global__ __launch_bounds__(kXThreadsFor<WT>) void xattn_lse_kernel(XattnArgs a) {
  using T = XTile<WT>;
  constexpr int kChunks = S * D / kXChunk;   // inner-dimension stages
  constexpr int kBk = 64 / S;                // reshaped columns per 64-token key block
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int h = lane >> 5;
  const int n = lane & 31;

  // Tile order: work-group L runs on XCD L % 8.  When B*H is a multiple of
  // 8, XCD x takes heads x, x+8, ...; within a head it walks bands of
  // kXBand row tiles, column tile by column tile, so the ~64 tiles resident
  // on one XCD share kXBand query strips and as many key strips in its L2.
  const int ntc = a.ntc, nrt = a.nrt;
  int bh, rt, ct;
  {
    const int L = blockIdx.x;
    const int per_head = nrt * ntc;
    int idx;
    if ((a.BH & 7) == 0) {
      const int k = L >> 3;
      bh = (L & 7) + 8 * (k / per_head);
      idx = k % per_head;
    } else {
      bh = L / per_head;
      idx = L % per_head;
    }
    const int band_tiles = kXBand * ntc;
    const int band = idx / band_tiles;
    const int rem = idx - band * band_tiles;
    const int rows_in_band = min(kXBand, nrt - band * kXBand);
    ct = rem / rows_in_band;
    rt = band * kXBand + (rem - ct * rows_in_band);
  }
  const int rq = a.Sq / S, rk = a.Sk / S;          // reshaped lengths
  const int past = (a.Sk - a.Sq) / S;             // reshaped causal offset
  const int r0 = rt * kXTileR, t0 = ct * T::kT;
  if (a.causal && t0 > r0 + kXTileR - 1 + past) return;   // the whole tile is masked

  const uint16_t* __restrict__ Kh = a.k + (int64_t)bh * a.Sk * D;
  const uint16_t* __restrict__ Qh = a.q + (int64_t)bh * a.Sq * D;

  // DMA: instruction kk of an operand tile covers its rows 8kk .. 8kk+7; lane
  // l fills LDS granule l % 8 of row 8kk + l / 8 with the source granule that
  // the swizzle puts there.  Wave w issues kk = w, w + 2 WT, ...: kIK of the
  // K' tile's T::kT / 8 and kIQ of the Q' tile's 16.
  constexpr int kIK = T::kT / 8 / T::kWaves, kIQ = kXTileR / 8 / T::kWaves;
  uint32_t voff_k[kIK], voff_q[kIQ];
#pragma unroll
  for (int i = 0; i < kIK; ++i) {
    const int row = 8 * (w + T::kWaves * i) + (lane >> 3);
    const int g = (lane & 7) ^ xswz(row);
    const int kr = min(t0 + row, rk - 1);   // rows past the end re-read the last (masked later)
    voff_k[i] = (uint32_t)(((int64_t)kr * S * D + 8 * g) * 2);
  }
#pragma unroll
  for (int i = 0; i < kIQ; ++i) {
    const int row = 8 * (w + T::kWaves * i) + (lane >> 3);
    const int g = (lane & 7) ^ xswz(row);
    const int qr = min(r0 + row, rq - 1);   // rows past the end are never stored
    voff_q[i] = (uint32_t)(((int64_t)qr * S * D + 8 * g) * 2);
  }
  // Stage c of K' is dimensions 64c .. 64c+63 of every K' row: byte 128c on.
  // Stage c of Q' is sub-row j = 64c / D taken in reverse (query row
  // r's + s-1-j), dimensions 64c % D on.
  auto issue = [&](int c, uint32_t stage) {
    const int j = (kXChunk * c) / D;
    const int d0 = (kXChunk * c) % D;
    const unsigned char* kb = (const unsigned char*)Kh + 128 * c;
    const unsigned char* qb = (const unsigned char*)Qh + (int64_t)((S - 1 - j) * D + d0) * 2;
    const uint32_t ka = lds0 + stage * T::kStageBytes + (uint32_t)w * 1024;
    const uint32_t qa = ka + T::kOpBytesK;
#pragma unroll
    for (int i = 0; i < kIK; ++i) dma16<0>(kb, voff_k[i], ka + i * T::kWaves * 1024);
#pragma unroll
    for (int i = 0; i < kIQ; ++i) dma16<0>(qb, voff_q[i], qa + i * T::kWaves * 1024);
  };

  // Wave (wt, wr): L^T rows (reshaped keys) 64 wt .. +63, columns (reshaped
  // queries) 64 wr .. +63, as 2 x 2 MFMA tiles.  Operand reads: lane reads
  // row n of a 32-row tile, inner dimensions 16 st + 8 h .. +7.
  const int wt = w >> 1, wr = w & 1;
  uint32_t aoff[2][4], boff[2][4];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int ra = 64 * wt + 32 * tt + n;
      const int rb = 64 * wr + 32 * tt + n;
      aoff[tt][st] = lds0 + (uint32_t)(ra * 128 + 16 * ((2 * st + h) ^ xswz(ra)));
      boff[tt][st] = lds0 + T::kOpBytesK + (uint32_t)(rb * 128 + 16 * ((2 * st + h) ^ xswz(rb)));
    }

  f32x16 acc[2][2];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) acc[tt][rr] = f32x16{};

  issue(0, 0);
  for (int c = 0; c < kChunks; ++c) {
    const uint32_t stage = (uint32_t)(c & 1) * T::kStageBytes;
    // This wave's loads of stage c are done and its reads of stage c-1 have
    // returned; after the barrier every wave is there, so stage c is in LDS
    // and the slot of stage c-1 is free for stage c+1, which then has the
    // whole of this stage's MFMA work to arrive.
    wait_vmem_lds0<0>();
    barrier_raw();
    if (c + 1 < kChunks) issue(c + 1, (uint32_t)((c + 1) & 1));
    // all 16 operand reads of the stage first, into distinct registers, so the
    // MFMAs wait on them progressively instead of on each read in turn
    u32x4 av[4][2], bv[4][2];
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        av[st][tt] = lds_read_b128(aoff[tt][st] + stage);
        bv[st][tt] = lds_read_b128(boff[tt][st] + stage);
      }
    __builtin_amdgcn_sched_barrier(0);   // keep the reads ahead of the MFMAs
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) acc[tt][rr] = mfma32(av[st][tt], bv[st][rr], acc[tt][rr]);
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- epilogue: per (reshaped row, key block) log2-sum-exp2 ----
  // acc[tt][rr] element v: key t' = t0 + 64 wt + 32 tt + 8 (v / 4) + 4 h + v % 4,
  // query r' = r0 + 64 wr + 32 rr + n.  A key block is kBk consecutive t'.
  // The scale is applied inside the exponent's fma (max of the raw sums, then
  // 2^(c acc - c max)); only a wave whose keys are not all visible to all its
  // rows (on the causal diagonal, or past the end of K) tests each key.
  const float c2 = a.scale_log2;
  float* __restrict__ out = a.lse + (int64_t)bh * rq * a.nbk;
  constexpr int kGroups = 32 / kBk;   // key blocks per 32-key MFMA tile
  const int wt0 = t0 + 64 * wt, wr0 = r0 + 64 * wr;
  const bool wave_masked = (wt0 + 63 > rk - 1) || (a.causal && wt0 + 63 > wr0 + past);
  auto epilogue = [&](auto masked_c) {
    constexpr bool kMasked = decltype(masked_c)::value;
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int r = wr0 + 32 * rr + n;
      const int lim = a.causal ? min(r + past, rk - 1) : rk - 1;   // last visible key
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int tb = wt0 + 32 * tt;
        float x[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          x[v] = acc[tt][rr][v];
          if constexpr (kMasked) {
            const int t = tb + 8 * (v >> 2) + 4 * h + (v & 3);
            if (t > lim) x[v] = -INFINITY;
          }
        }
        if constexpr (kBk == 4) {
          // 4 consecutive keys are one lane's v = 4u .. 4u+3: 4 groups per lane,
          // group index 2u + h
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const float m = fmaxf(fmaxf(x[4 * u], x[4 * u + 1]), fmaxf(x[4 * u + 2], x[4 * u + 3]));
            const float mc = m * c2;
            float e = 0.0f;
            if (!kMasked || m != -INFINITY) {
#pragma unroll
              for (int q = 0; q < 4; ++q) e += fast_exp2(fmaf(x[4 * u + q], c2, -mc));
            }
            const int kbk = tb / kBk + 2 * u + h;
            if (r < rq && kbk < a.nbk)
              out[(int64_t)r * a.nbk + kbk] = e > 0.0f ? mc + __log2f(e) : -INFINITY;
          }
        } else {
          // kBk = 8: group v / 4; kBk = 16: group v / 8 (both lane halves share groups)
          float mg[kGroups], eg[kGroups];
#pragma unroll
          for (int g = 0; g < kGroups; ++g) {
            mg[g] = -INFINITY;
            eg[g] = 0.0f;
          }
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int g = kBk == 8 ? (v >> 2) : (v >> 3);
            mg[g] = fmaxf(mg[g], x[v]);
          }
          float mcg[kGroups];
#pragma unroll
          for (int g = 0; g < kGroups; ++g) {
            mg[g] = max_with_half_swap(mg[g]);
            mcg[g] = mg[g] * c2;
          }
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int g = kBk == 8 ? (v >> 2) : (v >> 3);
            if (!kMasked || mg[g] != -INFINITY) eg[g] += fast_exp2(fmaf(x[v], c2, -mcg[g]));
          }
#pragma unroll
          for (int g = 0; g < kGroups; ++g) eg[g] = sum_with_half_swap(eg[g]);
          if (h == 0 && r < rq) {
#pragma unroll
            for (int g = 0; g < kGroups; ++g) {
              const int kbk = tb / kBk + g;
              if (kbk < a.nbk)
                out[(int64_t)r * a.nbk + kbk] = eg[g] > 0.0f ? mcg[g] + __log2f(eg[g]) : -INFINITY;
            }
          }
        }
      }
    }
  };
  if (wave_masked) epilogue(std::true_type{});
  else epilogue(std::false_type{});
}

// Wave-wide (64-lane) reductions.
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

constexpr int kMaxKeyBlocks = 1024;   // nbk limit of the block-sum and selection kernels

// One wave per (bh, query block): block sums of the reshaped softmax weights.
// Lane l handles key blocks l, l+64, ... (NU of them, 64 NU >= nbk).
template <int S, int NU>
__global__ __launch_bounds__(kWave) void xattn_blocksum_kernel(XattnArgs a) {
  constexpr int kBq = 64 / S;
  constexpr int kColsPerLane = NU;
  const int lane = threadIdx.x;
  const int bh = blockIdx.y;
  const int qi = blockIdx.x;
  const int rq = a.Sq / S;
  const int past = (a.Sk - a.Sq) / S;
  const int nbk = a.nbk;
  const int nu = (nbk + kWave - 1) / kWave;
  const float* __restrict__ lse = a.lse + (int64_t)bh * rq * nbk;
  float acc[kColsPerLane];
#pragma unroll
  for (int u = 0; u < kColsPerLane; ++u) acc[u] = 0.0f;
  const int rend = min(qi * kBq + kBq, rq);
  for (int r = qi * kBq; r < rend; ++r) {
    // key blocks this row can see at all (later ones were not written)
    const int kb_last = a.causal ? min((r + past) / kBq, nbk - 1) : nbk - 1;
    float v[kColsPerLane];
    float m = -INFINITY;
#pragma unroll
    for (int u = 0; u < kColsPerLane; ++u) {
      const int kb = u * kWave + lane;
      v[u] = (u < nu && kb <= kb_last) ? lse[(int64_t)r * nbk + kb] : -INFINITY;
      m = fmaxf(m, v[u]);
    }
    m = wave_max(m);   // finite: key 0 is visible to every row
    float s = 0.0f;
#pragma unroll
    for (int u = 0; u < kColsPerLane; ++u) s += fast_exp2(v[u] - m);
    s = wave_sum(s);
    const float norm = m + __log2f(s);
#pragma unroll
    for (int u = 0; u < kColsPerLane; ++u) acc[u] += fast_exp2(v[u] - norm);
  }
  float* __restrict__ out = a.block_sums + ((int64_t)bh * a.nbq + qi) * nbk;
#pragma unroll
  for (int u = 0; u < kColsPerLane; ++u) {
    const int kb = u * kWave + lane;
    if (u < nu && kb < nbk) out[kb] = acc[u];
  }
}

// 64-bit lane exchange with lane ^ j.
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t x, int j) {
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)x, j);
  const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(x >> 32), j);
  return ((uint64_t)hi << 32) | lo;
}

constexpr int kSelRows = 16;   // query-block rows per selection work-group, one wave each

template <int NU>
constexpr size_t selection_lds_bytes() {
  return (size_t)kSelRows * (kWave * NU + 1) * 4 * 2 + (size_t)kSelRows * (kWave * NU + 4);
}

// Selection by cumulative weight, kSelRows query-block rows per work-group.
// Wave w sorts row w: its order keys (forced columns at weight 0) go through
// a descending bitonic network over 64 * NU elements held in registers,
// element e = NU * lane + u in key[u] (distances below NU inside a lane,
// longer ones by lane exchange).  Then lane r of wave 0 runs row r's float64
// sums one term at a time: the total in column order and the ranked sums in
// rank order, from padded LDS copies of the values.  Each wave finally maps
// its row's rank positions back to columns.
template <int NU>
__global__ __launch_bounds__(kSelRows * kWave) void mask_cumulative_kernel(
    const float* __restrict__ sums, int64_t rows, int nbq, int nbk, float threshold, int keep_sink,
    int keep_diag, int causal, uint8_t* __restrict__ mask) {
  constexpr int N = kWave * NU;
  constexpr int LW = N + 1;   // padded row pitch (floats): lane-per-row reads hit distinct banks
  constexpr int LT = N + 4;   // padded row pitch of the take flags (bytes)
  extern __shared__ __attribute__((aligned(16))) unsigned char sel_smem[];
  float* vals = (float*)sel_smem;                  // [kSelRows][LW] weights, column order
  float* ranked = vals + kSelRows * LW;            // [kSelRows][LW] weights, rank order
  uint8_t* take = (uint8_t*)(ranked + kSelRows * LW);   // [kSelRows][LT]
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kSelRows + w;
  const bool valid = row < rows;
  const int i = (int)(row % nbq);
  const int diag = i + (nbk - nbq);   // query blocks are the last nbq of nbk
  auto forced = [&](int c) { return (keep_sink && c == 0) || (keep_diag && c == diag); };

  uint64_t key[NU];
  if (valid) {
    const float* __restrict__ x = sums + row * nbk;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int c = NU * lane + u;
      if (c < nbk) {
        const float v = x[c];
        vals[w * LW + c] = v;
        key[u] = rank_key(forced(c) ? 0.0f : v, c);
      } else {
        vals[w * LW + c] = 0.0f;   // the total's groups of 8 may reach past nbk
        key[u] = 0;                // below every real key: sorts last
      }
    }
    // bitonic sort, descending
#pragma unroll
    for (int k = 2; k <= N; k <<= 1) {
#pragma unroll
      for (int j = k >> 1; j > 0; j >>= 1) {
        if (j < NU) {
#pragma unroll
          for (int u = 0; u < NU; ++u) {
            const int p = u ^ j;
            if (p > u) {
              const bool desc = ((NU * lane + u) & k) == 0;
              const uint64_t a = key[u], b = key[p];
              // keys are distinct apart from the padding zeros, whose order
              // does not matter: one comparison decides either direction
              const bool swap = (a < b) == desc;
              key[u] = swap ? b : a;
              key[p] = swap ? a : b;
            }
          }
        } else {
          const int jl = j / NU;   // lane distance
          const bool lower = (lane & jl) == 0;
#pragma unroll
          for (int u = 0; u < NU; ++u) {
            const bool desc = ((NU * lane + u) & k) == 0;
            const uint64_t o = shfl_xor_u64(key[u], jl);
            const bool take_other = (o > key[u]) == (lower == desc);
            key[u] = take_other ? o : key[u];
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < NU; ++u) ranked[w * LW + NU * lane + u] = rank_key_score(key[u]);
  }
  __syncthreads();
  if (w == 0 && lane < kSelRows && (int64_t)blockIdx.x * kSelRows + lane < rows) {
    const float* vr = vals + lane * LW;
    const float* rr = ranked + lane * LW;
    uint8_t* tr = take + lane * LT;
    // Columns in groups of 8; the columns past nbk hold +0.0, which leaves
    // the sum (and every comparison with it) as it was.
    double total = 0.0;
    for (int c0 = 0; c0 < nbk; c0 += 8) {
      float t[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) t[q] = vr[c0 + q];
#pragma unroll
      for (int q = 0; q < 8; ++q) total += (double)t[q];
    }
    const double required = (double)threshold * total;
    // Ranks in groups of 8 without per-rank branches: ranks past nbk hold the
    // padding keys (sorted last), so their flags and the sum after them are
    // never read.  N is a multiple of 8, so a group never leaves the row.
    double before = 0.0;
    for (int p0 = 0; p0 < nbk; p0 += 8) {
      float t[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) t[q] = rr[p0 + q];
      uint32_t f[2] = {0u, 0u};
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        f[q >> 2] |= (before < required ? 1u : 0u) << (8 * (q & 3));
        before += (double)t[q];
      }
      *(uint32_t*)(tr + p0) = f[0];
      *(uint32_t*)(tr + p0 + 4) = f[1];
    }
  }
  __syncthreads();
  if (valid) {
    uint8_t* __restrict__ out = mask + row * nbk;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int e = NU * lane + u;
      if (e < nbk) {
        const int c = rank_key_column(key[u]);
        bool sel = take[w * LT + e] != 0 || forced(c);
        if (causal && c > diag) sel = false;
        out[c] = sel ? 1 : 0;
      }
    }
  }
}

template <int D, int S>
hipError_t launch_xattn_ds(const XattnArgs& a, hipStream_t stream) {
  const int64_t tiles = (int64_t)a.BH * a.nrt * a.ntc;
  if (tiles > 0x7fffffffLL) return hipErrorInvalidValue;
  using T = XTile<kXWT>;
  auto kern = xattn_lse_kernel<D, S, kXWT>;
  if (T::kLdsBytes > 64 * 1024) {
    static DeviceHighWater lds_set;   // per instantiation and device
    hipError_t e = lds_set.raise_to((int)T::kLdsBytes, [&](int v) {
      return hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, v);
    });
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)tiles), dim3(T::kThreads), T::kLdsBytes, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)a.nbq, (unsigned)a.BH);
  if (a.nbk <= 64) hipLaunchKernelGGL((xattn_blocksum_kernel<S, 1>), grid, dim3(kWave), 0, stream, a);
  else if (a.nbk <= 128) hipLaunchKernelGGL((xattn_blocksum_kernel<S, 2>), grid, dim3(kWave), 0, stream, a);
  else if (a.nbk <= 256) hipLaunchKernelGGL((xattn_blocksum_kernel<S, 4>), grid, dim3(kWave), 0, stream, a);
  else if (a.nbk <= 512) hipLaunchKernelGGL((xattn_blocksum_kernel<S, 8>), grid, dim3(kWave), 0, stream, a);
  else hipLaunchKernelGGL((xattn_blocksum_kernel<S, 16>), grid, dim3(kWave), 0, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_xattn_d(const XattnArgs& a, hipStream_t stream) {
  switch (a.stride) {
    case 4: return launch_xattn_ds<D, 4>(a, stream);
    case 8: return launch_xattn_ds<D, 8>(a, stream);
    case 16: return launch_xattn_ds<D, 16>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int xattn_max_key_blocks() { return kMaxKeyBlocks; }

size_t xattn_lse_bytes(int B, int H, int Sq, int Sk, int stride) {
  const size_t nbk = (size_t)(Sk + kBlock - 1) / kBlock;
  return (size_t)B * H * (size_t)(Sq / stride) * nbk * sizeof(float);
}

hipError_t launch_xattn_block_sums(XattnArgs a, hipStream_t stream) {
  a.ntc = ((a.Sk / a.stride) + XTile<kXWT>::kT - 1) / XTile<kXWT>::kT;
  a.nrt = ((a.Sq / a.stride) + kXTileR - 1) / kXTileR;
  return a.D == 64 ? launch_xattn_d<64>(a, stream) : launch_xattn_d<128>(a, stream);
}

template <int NU>
hipError_t launch_cumulative_nu(const float* sums, int64_t rows, int nbq, int nbk, float threshold,
                                int keep_sink, int keep_diag, int causal, uint8_t* mask,
                                hipStream_t stream) {
  constexpr size_t lds = selection_lds_bytes<NU>();
  auto kern = mask_cumulative_kernel<NU>;
  if (lds > 64 * 1024) {
    static DeviceHighWater lds_set;   // per instantiation and device
    hipError_t e = lds_set.raise_to((int)lds, [&](int v) {
      return hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, v);
    });
    if (e != hipSuccess) return e;
  }
  const int64_t groups = (rows + kSelRows - 1) / kSelRows;
  hipLaunchKernelGGL(kern, dim3((unsigned)groups), dim3(kSelRows * kWave), lds, stream, sums, rows,
                     nbq, nbk, threshold, keep_sink, keep_diag, causal, mask);
  return hipGetLastError();
}

hipError_t launch_mask_cumulative(const float* sums, int B, int H, int nbq, int nbk, float threshold,
                                  int keep_sink, int keep_diag, int causal, uint8_t* mask,
                                  hipStream_t stream) {
  const int64_t rows = (int64_t)B * H * nbq;
  if (nbk <= 64)
    return launch_cumulative_nu<1>(sums, rows, nbq, nbk, threshold, keep_sink, keep_diag, causal, mask, stream);
  if (nbk <= 128)
    return launch_cumulative_nu<2>(sums, rows, nbq, nbk, threshold, keep_sink, keep_diag, causal, mask, stream);
  if (nbk <= 256)
    return launch_cumulative_nu<4>(sums, rows, nbq, nbk, threshold, keep_sink, keep_diag, causal, mask, stream);
  if (nbk <= 512)
    return launch_cumulative_nu<8>(sums, rows, nbq, nbk, threshold, keep_sink, keep_diag, causal, mask, stream);
  return launch_cumulative_nu<16>(sums, rows, nbq, nbk, threshold, keep_sink, keep_diag, causal, mask, stream);
}

}  // namespace bsattn
