// Block-sparse attention forward (prefill) for gfx950.
//
// What is computed follows the TileLang block-sparse Flash-Attention guide,
// §4.3–§4.7: one work item per (batch, head, 64-row query block); only the
// key blocks its mask row selects are visited (§4.4), the diagonal block is
// masked causally (§4.5), the softmax is carried online in base 2 with the
// scale D^-1/2 * log2(e) folded into one multiply-add (§4.6), probabilities
// are rounded to bfloat16 for the P.V product, and the result is divided by
// the running sum at the end (§4.7).
//
// How it is mapped to CDNA4 (this is not the guide's kernel design):
// * Two or four wave64s per work item.  Waves w and w^1 take query rows
//   0..31 and 32..63.  With two waves (KS = 1: D = 64 when the items fill
//   the GPU) each sees all 64 keys of a block; with four (KS = 2: always at
//   D = 128, and at D = 64 when the items fit in one round of resident
//   work-groups) wave w also takes keys 32 (w >> 1) .. +31 only, the two key
//   halves run as independent online softmaxes and are merged once per item
//   through LDS.  Splitting the keys halves the per-wave registers (two waves
//   per SIMD at D = 128 instead of one) without reading the K/V tiles from
//   LDS more than once per query row.
// * Scores are formed transposed, S^T = K . Q^T, with v_mfma_f32_32x32x16_bf16:
//   the accumulator gives each lane ONE query row (lane % 32) and 16 of the
//   wave's 32 keys, so the row max / row sum are in-lane reductions plus a
//   single permlane32 swap, and the exponentiated scores are already laid out
//   as the B operand of O^T = V^T . P^T (no LDS round trip for P).
// * Software pipeline over the active blocks t = 0, 1, ...: while the VALU
//   works on the softmax of block t, the matrix cores run P.V of block t-1
//   and Q.K^T of block t+1.
// * The mask row is compacted once, at the start, into the ascending list of
//   key blocks in LDS (64-column ballots); a block whose keys are not all
//   visible to every row (on the causal diagonal, or past the end of K) is
//   masked when its scores come up.
// * Queries may be fewer than keys (Sq <= Sk): they are then the last Sq
//   positions, and the causal rule compares key t with row + Sk - Sq (the
//   TileLang FlashAttention guide's BHSD example, past_len; the block-sparse
//   guide's §8 Triton reference, PAST_LEN).
// * K and V tiles travel HBM -> LDS with global_load_lds_dwordx4 (no
//   registers) into two-slot rings, one block ahead, with explicit vmcnt
//   waits.  Rows are XOR-swizzled in 16-byte granules so the K reads
//   (ds_read_b128) and the transposed V reads (ds_read_b64_tr_b16) are free
//   of bank conflicts; every LDS address is a per-lane constant plus an
//   immediate.
// * Work items are issued heaviest-first (last query block first), and when
//   batch*heads is a multiple of 8 each head's items stay on one XCD so its
//   K/V stay in that XCD's L2 (item_order.hpp).
// * Long causal rows (more than split_min key blocks, when the caller gives a
//   workspace) run as two halves in two work-groups; each leaves fp32 rows
//   plus (row max, row sum), and a small merge launch combines them by the
//   log-sum-exp rule of the split-KV decode (TileLang block-sparse guide,
//   §6.2), so a few dense rows do not hold up the whole launch.
#include <math.h>

#include <algorithm>

#include <type_traits>

#include "common.hpp"
#include "item_order.hpp"
#include "launch.hpp"

namespace bsattn {

namespace {


template <int KS>
constexpr int kThreadsFor = 2 * KS * kWave;

// KS: key splits per work item.  KS = 1: two waves, each 32 query rows x all
// 64 keys of a block.  KS = 2: four waves, each 32 query rows x 32 keys.
template <int D, int KS>
struct Cfg {
  static constexpr int kWaves = 2 * KS;
  static constexpr int kThreads = kThreadsFor<KS>;
  static constexpr int NT = 2 / KS;                     // 32-key score tiles per wave and block
  static constexpr int G = D / 8;                       // 16-byte granules per row
  static constexpr int kRowBytes = D * 2;
  static constexpr int kTileBytes = 64 * kRowBytes;     // one K or V tile
  static constexpr int kTileInstr = kTileBytes / 1024;  // 1 KiB wave-wide DMAs per tile
  static constexpr int kWaveInstr = kTileInstr / kWaves;  // per wave, per tile
  static constexpr int kRowsPerInstr = 1024 / kRowBytes;
  static constexpr int kRingBytes = 4 * kTileBytes;     // K slots 0, 1, then V slots 0, 1
  static constexpr int kSteps = D / 16;                 // k-steps of S^T = K . Q^T
  static constexpr int kDT = D / 32;                    // 32-row tiles of O^T
  static constexpr int kXchgBytes = kDT / 2 * 16 * kWave * 4;  // o half-tiles one wave hands over
  static_assert(KS == 1 || kWaves * kXchgBytes <= 2 * kTileBytes, "exchange fits the K slots");
  static constexpr int kStatsBytes = KS == 2 ? kWaves * kWave * 8 : 0;
};

// 16-byte granule swizzles: logical granule g of tile row r is stored at
// granule g ^ swz(r).  K's depends on r & 15 only, V's on r & 3 only.
template <int D>
__device__ __forceinline__ int swz_k(int r) {
  return D == 64 ? ((r >> 1) & 7) : (r & 15);
}
template <int D>
__device__ __forceinline__ int swz_v(int r) {
  return D == 64 ? ((r & 2) << 1) : ((r & 3) << 2);
}


// Calls f(integral_constant<int, K>) for K = 0, 1, ... in order.
template <class F, int... Ks>
__device__ __forceinline__ void static_for(std::integer_sequence<int, Ks...>, F&& f) {
  (f(std::integral_constant<int, Ks>{}), ...);
}

template <int D, int KS>
size_t lds_bytes(int nb) {
  using C = Cfg<D, KS>;
  // the K/V rings, the row statistics of the key-half merge (KS = 2: 4 waves
  // x 64 lanes x 2 floats), then the block list (nb entries + its length),
  // 16-byte aligned
  return (size_t)C::kRingBytes + C::kStatsBytes + (size_t)(((nb + 1) * 2 + 15) / 16) * 16;
}

// The staged output tile: row r's 16-byte granule g sits at granule
// g ^ swz_k(r) of the row, with its two 8-byte halves swapped in the rows
// staged_swap marks, so both the per-lane 8-byte writes (one granule half
// per lane, 32 rows per instruction) and the 16-byte reads of whole rows
// are free of bank conflicts (checked against a 32- and a 64-bank model).
template <int D>
__device__ __forceinline__ int staged_swap(int r) {
  return D == 128 ? ((r >> 3) ^ (r >> 4)) & 1 : (r ^ (r >> 4)) & 1;
}
template <int D>
__device__ __forceinline__ u32x4 staged_row_piece(const unsigned char* tile, int r, int g) {
  const u32x4 v = *(const u32x4*)(tile + r * (D * 2) + (g ^ swz_k<D>(r)) * 16);
  return staged_swap<D>(r) ? u32x4{v[2], v[3], v[0], v[1]} : v;
}

// S^T of one block for one wave: NT tiles of 32 keys x its 32 query rows.
template <int NT>
struct Scores {
  f32x16 s[NT];
};
// P^T of one block as bf16 B operands of the wave's 2 NT 16-key P.V steps.
template <int NT>
struct Probs {
  u32x4 p[2 * NT];
};


constexpr int kMaxKeyChunks = 4;   // fused row selection handles up to 256 key blocks

template <int D, int KS, bool CAUSAL, int SRC>
__global__ __launch_bounds__(kThreadsFor<KS>) void prefill_kernel(PrefillArgs a, ItemOrder items,
                                                                  ItemOrder helpers) {
  using C = Cfg<D, KS>;
  constexpr int kWaves = C::kWaves;
  constexpr int NT = C::NT;
  using Sc = Scores<NT>;
  using Pr = Probs<NT>;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  float* stats = (float*)(smem + C::kRingBytes);                    // [wave][m | l][lane]
  uint16_t* list = (uint16_t*)(smem + C::kRingBytes + C::kStatsBytes);

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
  const int rg = w & 1;      // query rows 32 rg .. +31
  const int kh = w >> 1;     // keys 32 NT kh .. +32 NT - 1 of every block
  const int lane = tid & 63;
  const int h = lane >> 5;   // which half of the key rows / k-group this lane holds
  const int n = lane & 31;   // query row within the wave's 32

  const int nbq = a.nbq, nbk = a.nbk;
  const int Sq = a.Sq, Sk = a.Sk;
  const int past = Sk - Sq;   // query row r sits at key position r + past
  int bh, i;
  // Work-groups below n_help take the second half of a long row's list (the
  // query blocks i >= split_row0, heaviest first); the rest are the items.
  // The mask-row and block-score sources split (every work-group of a row
  // builds the same list); a given list never does, whatever split_min says.
  constexpr bool kCanSplit = SRC != kSrcList;
  const int n_help =
      (kCanSplit && a.split_min > 0) ? a.B * a.H * (nbq - a.split_row0) : 0;
  const bool helper = (int)blockIdx.x < n_help;
  if (helper) {
    map_item(helpers, blockIdx.x, bh, i);
    i += a.split_row0;
  } else {
    map_item(items, (int)blockIdx.x - n_help, bh, i);
  }

  const int64_t q_off = (int64_t)bh * Sq * D;
  const int64_t kv_off = (int64_t)bh * Sk * D;
  const uint16_t* __restrict__ Q = a.q + q_off;
  const uint16_t* __restrict__ K = a.k + kv_off;
  const uint16_t* __restrict__ V = a.v + kv_off;
  const int q0 = i * 64;
  const int qrow = q0 + 32 * rg + n;
  // Key blocks past the last one any row of this query block can see are skipped.
  const int lim = CAUSAL ? min(nbk, ((q0 + 63 + past) >> 6) + 1) : nbk;
  // A key block needs masking inside the block when some of its keys lie
  // after the first query row's position (causal), or past the end of K.
  auto needs_mask = [&](int j) {
    return (CAUSAL && j * 64 + 63 > q0 + past) || (j * 64 + 64 > Sk);
  };

  // The mask row's first 256 bytes are requested before Q, so the list can be
  // built (and the first K/V tiles requested) while Q is still on its way.
  // (Unconditional loads at a clamped column keep the compiler from waiting
  // on each; columns past lim are ignored when the list is built.)
  // The fused forms do the same with the block-score row (nb <= 256).
  uint8_t mpre[kMaxKeyChunks];
  float xpre[kMaxKeyChunks];
  if constexpr (SRC == kSrcMask) {
    const uint8_t* mrow = a.mask + ((int64_t)bh * nbq + i) * nbk;
#pragma unroll
    for (int u = 0; u < kMaxKeyChunks; ++u) mpre[u] = mrow[min(kWave * u + lane, lim - 1)];
    asm volatile("" ::: "memory");   // issued before the Q loads below
  } else if constexpr (SRC == kSrcTopk || SRC == kSrcThreshold) {
    const float* xrow = a.scores + ((int64_t)bh * nbk + i) * nbk;
#pragma unroll
    for (int u = 0; u < kMaxKeyChunks; ++u) xpre[u] = xrow[min(kWave * u + lane, nbk - 1)];
    asm volatile("" ::: "memory");   // issued before the Q loads below
  }

  // Q^T as the B operand of S^T = K . Q^T: lane holds row qrow, dims 16s + 8h .. +8.
  // (A helper loads it only once it knows its row is long.)
  u32x4 qf[C::kSteps];
  auto load_q = [&]() {
    const int qr = min(qrow, Sq - 1);   // rows past the end are never stored
#pragma unroll
    for (int s = 0; s < C::kSteps; ++s)
      qf[s] = *(const u32x4*)(Q + (int64_t)qr * D + 16 * s + 8 * h);
  };
  if (!helper) load_q();

  // ---- this query block's list of key blocks, ascending, into LDS ----
  // From a mask row, a given list, or (fused) a block-score row: the row is
  // selected here as the mask builders select it (TileLang block-sparse guide
  // §3.1 top-k, §3.2 threshold: optional dense last two rows, tril, then the
  // forced diagonal of the XAttention guide), written out if asked, and
  // compacted in the same pass.
  // Fused forms: the selected columns of the row, one bit each, written to the
  // mask output after the forward pass so the stores stay off the first waits.
  uint64_t selbits[kMaxKeyChunks] = {};
  if (w == 0) {
    int count = 0;
    const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    if constexpr (SRC == kSrcList) {
      const int64_t row = (int64_t)bh * nbq + i;
      const int nl = max(0, min(a.cnt[row], nbk));
      const int32_t* src = a.idx + row * nbk;
      for (int c0 = 0; c0 < nl; c0 += kWave) {
        const int p = c0 + lane;
        const int j = p < nl ? src[p] : -1;
        const bool ok = j >= 0 && j < lim;
        const uint64_t bits = wave_ballot(ok);
        if (ok) list[count + __popcll(bits & below)] = (uint16_t)j;
        count += __popcll(bits);
      }
    } else if constexpr (SRC == kSrcMask) {
      const uint8_t* mrow = a.mask + ((int64_t)bh * nbq + i) * nbk;
#pragma unroll
      for (int u = 0; u < kMaxKeyChunks; ++u) {
        if (kWave * u >= lim) break;
        const int j = kWave * u + lane;
        const bool ok = j < lim && mpre[u] != 0;
        const uint64_t bits = wave_ballot(ok);
        if (ok) list[count + __popcll(bits & below)] = (uint16_t)j;
        count += __popcll(bits);
      }
      for (int c0 = kWave * kMaxKeyChunks; c0 < lim; c0 += kWave) {   // rows past 256 blocks
        const int j = c0 + lane;
        const bool ok = j < lim && mrow[j] != 0;
        const uint64_t bits = wave_ballot(ok);
        if (ok) list[count + __popcll(bits & below)] = (uint16_t)j;
        count += __popcll(bits);
      }
    } else {
      // square problem: nbq = nbk = nb; the score row is in xpre (loaded above)
      const bool dense_row = a.dense2 && i >= nbk - 2;
      const bool all = dense_row || (SRC == kSrcTopk && a.topk >= nbk);
      const bool none = SRC == kSrcTopk && a.topk == 0 && !dense_row;
      const bool ranked = SRC == kSrcTopk && !all && !none;
      // Top-k by a bitwise radix select over the wave (wave_topk_cut): the
      // row's order keys (distinct: ties are broken by the column) sit in
      // registers, lane l holding columns l, l+64, ...
      uint64_t key[kMaxKeyChunks];
      uint64_t hm = 0, prefix = 0;
      if (ranked) {
#pragma unroll
        for (int u = 0; u < kMaxKeyChunks; ++u) {
          const int c = 64 * u + lane;
          key[u] = c < nbk ? rank_key(xpre[u], c) : 0ull;   // 0 is below every real key
        }
        wave_topk_cut(key, (nbk + kWave - 1) / kWave, a.topk, hm, prefix);
      }
#pragma unroll
      for (int u = 0; u < kMaxKeyChunks; ++u) {
        const int j = 64 * u + lane;
        if (64 * u >= nbk) break;
        bool sel = false;
        if (j < nbk && j <= i) {   // tril: columns above the diagonal are never selected
          if (all) sel = true;
          else if (SRC == kSrcThreshold) sel = dense_row || xpre[u] > a.threshold;
          else if (ranked) sel = (key[u] & hm) >= prefix;
          if (a.diag && j == i) sel = true;
        }
        selbits[u] = wave_ballot(sel);
        const bool ok = sel && j < lim;
        const uint64_t bits = wave_ballot(ok);
        if (ok) list[count + __popcll(bits & below)] = (uint16_t)j;
        count += __popcll(bits);
      }
    }
    if (lane == 0) list[nbk] = (uint16_t)count;   // the slot after the list holds its length
  }
  __syncthreads();
  int nblk = __builtin_amdgcn_readfirstlane((int)list[nbk]);
  // A long row: the item takes the first half of the list, its helper the
  // second; a helper whose row is not long has nothing to do.
  int part = -1;   // -1: the whole row, written to out
  int64_t slot = 0;
  if constexpr (kCanSplit) {
    if (a.split_min > 0 && i >= a.split_row0) {
      slot = (int64_t)bh * (nbq - a.split_row0) + (i - a.split_row0);
      const bool split = nblk > a.split_min;
      if (!helper && tid == 0) a.part_flag[slot] = split ? 1 : 0;
      if (!split && helper) return;
      if (split) {
        const int first = nblk >> 1;
        if (helper) {
          load_q();
          part = 1;
          list += first;
          nblk -= first;
        } else {
          part = 0;
          nblk = first;
        }
      }
    }
  }

  // ---- per-lane DMA source byte offsets for this wave's share of a tile ----
  // Instruction kk covers tile rows kk*kRowsPerInstr .. +kRowsPerInstr-1; lane l
  // fills stored granule l % G of row kk*kRowsPerInstr + l / G.
  uint32_t dma_k[C::kWaveInstr], dma_v[C::kWaveInstr];
  int dma_r[C::kWaveInstr];
#pragma unroll
  for (int q = 0; q < C::kWaveInstr; ++q) {
    const int kk = w + kWaves * q;
    const int r = kk * C::kRowsPerInstr + lane / C::G;
    const int sg = lane % C::G;
    dma_r[q] = r;
    dma_k[q] = (uint32_t)((r * D + (sg ^ swz_k<D>(r)) * 8) * 2);
    dma_v[q] = (uint32_t)((r * D + (sg ^ swz_v<D>(r)) * 8) * 2);
  }
  const uint32_t wbase = lds0 + (uint32_t)w * 1024;   // this wave's instructions: kk = w + kWaves q
  // Load this wave's share of key block j's K (or V) tile into ring slot kSlot.
  auto issue = [&](auto slot_c, auto is_v, int jv) {
    constexpr uint32_t kSlot = decltype(slot_c)::value;
    constexpr bool kV = decltype(is_v)::value;
    const int j = __builtin_amdgcn_readfirstlane(jv);
    const uint16_t* base = (kV ? V : K) + (int64_t)j * 64 * D;
    const int last = Sk - 1 - j * 64;
    if (last >= 63) {
#pragma unroll
      for (int q = 0; q < C::kWaveInstr; ++q)
        dma16<kSlot>(base, kV ? dma_v[q] : dma_k[q], wbase + q * kWaves * 1024);
    } else {
      // ragged last block: rows past the end re-read the last row (masked later)
#pragma unroll
      for (int q = 0; q < C::kWaveInstr; ++q) {
        const uint32_t back = (uint32_t)(max(dma_r[q] - last, 0) * D * 2);
        dma16<kSlot>(base, (kV ? dma_v[q] : dma_k[q]) - back, wbase + q * kWaves * 1024);
      }
    }
  };
  using K0 = std::integral_constant<uint32_t, 0 * C::kTileBytes>;
  using K1 = std::integral_constant<uint32_t, 1 * C::kTileBytes>;
  using V0 = std::integral_constant<uint32_t, 2 * C::kTileBytes>;
  using V1 = std::integral_constant<uint32_t, 3 * C::kTileBytes>;
  using IsK = std::false_type;
  using IsV = std::true_type;

  // ---- per-lane LDS read addresses (bytes, slot 0 of the ring) ----
  // K rows of this wave's keys (tile tt adds 32 rows); V^T rows of its 16-key steps.
  uint32_t koff[C::kSteps];
#pragma unroll
  for (int st = 0; st < C::kSteps; ++st) {
    const int r = 32 * NT * kh + n;
    koff[st] = lds0 + (uint32_t)((r * C::G + ((2 * st + h) ^ swz_k<D>(r))) * 16);
  }
  const int tr_r = (lane >> 2) & 3;
  const int tr_m = lane & 3;
  const int tr_g = (lane >> 4) & 1;
  uint32_t voff[C::kDT];
#pragma unroll
  for (int t = 0; t < C::kDT; ++t) {
    const int gran = 4 * t + 2 * tr_g + (tr_m >> 1);
    voff[t] = lds0 + (uint32_t)(((32 * NT * kh + 4 * h + tr_r) * C::G + (gran ^ swz_v<D>(tr_r))) *
                                    16 +
                                (tr_m & 1) * 8);
  }

  f32x16 o[C::kDT];
#pragma unroll
  for (int t = 0; t < C::kDT; ++t) o[t] = f32x16{};
  // m: the exponent offset in use for this lane's row (always finite; 0 until
  // a block shows the row a finite score); l: the running row sum.
  float m = 0.0f;
  float l = 0.0f;
  const float c = (float)(1.4426950408889634 / __builtin_sqrt((double)D));

  // ---- the phases of one block ----
  // S^T of the block whose K tile sits in slot kSlot.
  auto qk = [&](auto slot_c, Sc& sc) {
    constexpr uint32_t kSlot = decltype(slot_c)::value;
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) sc.s[tt] = f32x16{};
#pragma unroll
    for (int st = 0; st < C::kSteps; ++st)
#pragma unroll
      for (int tt = 0; tt < NT; ++tt)
        sc.s[tt] = mfma32(lds_read_b128(koff[st] + kSlot + tt * 32 * C::G * 16), qf[st], sc.s[tt]);
  };
  // O^T += V^T . P^T for the block whose V tile sits in slot kSlot.
  auto pv = [&](auto slot_c, const Pr& pr) {
    constexpr uint32_t kSlot = decltype(slot_c)::value;
#pragma unroll
    for (int u = 0; u < 2 * NT; ++u) {
#pragma unroll
      for (int tt = 0; tt < C::kDT; ++tt) {
        const uint32_t a0 = voff[tt] + kSlot + (16 * u) * C::G * 16;
        const u32x2 lo = lds_read_tr16(a0);
        const u32x2 hi = lds_read_tr16(a0 + 8 * C::G * 16);
        o[tt] = mfma32(u32x4{lo[0], lo[1], hi[0], hi[1]}, pr.p[u], o[tt]);
      }
    }
  };
  // In-block masking of key block j: keys past the end of K, and (causal)
  // keys after the query row's position, get -inf.
  auto mask_block = [&](int j, Sc& sc) {
    const int kbase = j * 64 + 32 * NT * kh;
    int vis = Sk - kbase;
    if (CAUSAL) vis = min(vis, qrow + past - kbase + 1);
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
      for (int ii = 0; ii < 16; ++ii) {
        const int k0 = 32 * tt + 8 * (ii >> 2) + 4 * h + (ii & 3);
        if (k0 >= vis) sc.s[tt][ii] = -INFINITY;
      }
  };
  // Softmax of one block: P = 2^(S c - m c) packed to bf16 B operands of
  // P.V, and the row sum taken over the packed values with v_dot2 (two per
  // instruction, and the same values P.V multiplies).  The running max m
  // only serves as the exponent offset, so it is moved lazily: a block's
  // exponentials are first taken against the current m, and only when some
  // lane's 16 NT-term partial sum exceeds 2^8 (so some probability may have
  // reached that size) is m raised to the row maxima, o and l rescaled and
  // the block's exponentials taken again.  A first pass against a stale m
  // can overflow only when the redo is taken, which discards it.  The first
  // block of an item sets m from its row maxima directly.
  constexpr float kLazySum = 256.0f;   // 2^8
  const uint32_t ones = 0x3F803F80u;   // bf16 (1, 1)
  auto dot_sum = [&](uint32_t pk, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk),
                                           __builtin_bit_cast(bf16x2, ones), acc, false);
  };
  auto exps = [&](const Sc& sc, Pr& pr, float mc) -> float {
    float rs = 0.0f;
#pragma unroll
    for (int u = 0; u < 2 * NT; ++u) {
      const f32x16& sp = sc.s[u >> 1];
      const int base = 8 * (u & 1);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t pk = pack_bf16x2(fast_exp2(fmaf(sp[base + 2 * k], c, -mc)),
                                        fast_exp2(fmaf(sp[base + 2 * k + 1], c, -mc)));
        pr.p[u][k] = pk;
        rs = dot_sum(pk, rs);
      }
    }
    return rs;
  };
  auto row_max = [&](const Sc& sc) {
    float mx = sc.s[0][0];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
      for (int ii = (tt == 0 ? 1 : 0); ii < 16; ++ii) mx = fmaxf(mx, sc.s[tt][ii]);
    return max_with_half_swap(mx);
  };
  // Raise m to the block's row maxima, rescale o and l, redo the exponentials.
  auto raise = [&](const Sc& sc, Pr& pr) -> float {
    const float m_new = fmaxf(m, row_max(sc));   // a fully masked row keeps its m
    const float alpha = fast_exp2((m - m_new) * c);
    l *= alpha;
#pragma unroll
    for (int tt = 0; tt < C::kDT; ++tt)
#pragma unroll
      for (int ii = 0; ii < 16; ++ii) o[tt][ii] *= alpha;
    m = m_new;
    return exps(sc, pr, m * c);
  };
  // First block of an item: m = row max (0 for a row it fully masks).
  auto softmax_first = [&](const Sc& sc, Pr& pr) {
    const float mx = row_max(sc);
    m = (mx == -INFINITY) ? 0.0f : mx;
    l = exps(sc, pr, m * c);
  };
  // Any later block, outside the pipelined loop.
  auto softmax = [&](const Sc& sc, Pr& pr) {
    float rs = exps(sc, pr, m * c);
    // keep the first pass ahead of the redo test
#pragma unroll
    for (int u = 0; u < 2 * NT; ++u) asm volatile("" ::"v"(pr.p[u]));
    asm volatile("" ::"v"(rs));
    if (wave_ballot(rs > kLazySum) != 0) rs = raise(sc, pr);
    l += rs;
  };
  // ---- software pipeline over the list ----
  // Block t's K tile goes to K slot t&1 and its V tile to V slot t&1.
  // Iteration t: wait + barrier (K_{t+1}, V_{t-1} landed; every wave is done
  // with K_t and V_{t-2}); load V_t and K_{t+2}; then
  //   P.V of block t-1 | Q.K^T of block t+1 | exp of block t.
  // In the iteration with no K_{t+2} to load, the last block's V tile goes
  // into that free K slot instead, one iteration early, so the last block
  // does not wait for its own V load.
  Sc sa, sb;
  Pr pa, pb;
  if (nblk > 0) {
    issue(K0{}, IsK{}, list[0]);
    issue(V0{}, IsV{}, list[0]);
    if (nblk > 1) {
      issue(K1{}, IsK{}, list[1]);
      wait_vmem<2 * C::kWaveInstr>();   // K_0 landed (V_0 and K_1 may still be in flight)
    } else {
      wait_vmem<C::kWaveInstr>();
    }
    barrier_raw();
    qk(K0{}, sa);
  }

  // One steady-state iteration, 1 <= t <= nblk - 2 (block t needs no masking).
  // Hand-ordered as kSlots MFMA slots, each
  //   { LDS operand read for slot k+kAhead ; MFMA k ; softmax slice k },
  // fenced so the compiler keeps the order: the matrix cores run P.V of
  // block t-1 and Q.K^T of block t+1 while the VALU takes the exponentials
  // of block t (against the current running max; see softmax above).
  constexpr int kPvMfma = 2 * NT * C::kDT;   // u-major, tile-minor
  constexpr int kQkMfma = NT * C::kSteps;    // step-major, tile-minor
  constexpr int kSlots = kPvMfma + kQkMfma;
  constexpr int kPerSlot = 16 * NT / kSlots; // score elements per lane per slot
  static_assert(kPerSlot * kSlots == 16 * NT, "slices cover the block");
#ifndef BSATTN_AHEAD
#define BSATTN_AHEAD 2
#endif
  constexpr int kAhead = BSATTN_AHEAD;       // LDS operand reads issued this many slots ahead
  // At D = 128 the iteration's two tile loads go out in two bursts: V right
  // after the barrier, K after the last P.V slot (K_{t+2} is first read one
  // iteration later).  A work-group's 32 KiB in one burst measured 3-4%
  // slower at B4 H32 S8192; at D = 64 the split made no difference.
  constexpr int kKIssueSlot = D == 128 ? kPvMfma - 1 : -1;
  auto steady = [&](auto kt, auto kn, auto vt, auto vp, int t, Sc& s_cur, Sc& s_next,
                    const Pr& p_prev, Pr& p_cur) {
    constexpr uint32_t kN = decltype(kn)::value;
    constexpr uint32_t kVP = decltype(vp)::value;
    // Both list entries are read before the wait and the barrier, so their
    // LDS round trips overlap the wait.
    const int jt = __builtin_amdgcn_readfirstlane((int)list[t]);
    const int jn = __builtin_amdgcn_readfirstlane((int)list[t + 2 < nblk ? t + 2 : t + 1]);
    wait_vmem<0>();
    barrier_raw();
    issue(vt, IsV{}, jt);
    auto issue_k = [&]() {
      if (t + 2 < nblk) issue(kt, IsK{}, jn);
      else issue(kt, IsV{}, jn);   // the last block's V, into the K slot nothing needs
    };
    if constexpr (kKIssueSlot < 0) issue_k();
    if (needs_mask(jt)) mask_block(jt, s_cur);

    u32x4 op[kSlots];
    auto read = [&](auto k_c) {
      constexpr int k = decltype(k_c)::value;
      if constexpr (k < kPvMfma) {
        constexpr int u = k / C::kDT, tt = k % C::kDT;
        const uint32_t a0 = voff[tt] + kVP + (16 * u) * C::G * 16;
        const u32x2 lo = lds_read_tr16(a0);
        const u32x2 hi = lds_read_tr16(a0 + 8 * C::G * 16);
        op[k] = u32x4{lo[0], lo[1], hi[0], hi[1]};
      } else {
        constexpr int kk = k - kPvMfma, st = kk / NT, tile = kk % NT;
        op[k] = lds_read_b128(koff[st] + kN + tile * 32 * C::G * 16);
      }
    };
    auto mfma = [&](auto k_c) {
      constexpr int k = decltype(k_c)::value;
      if constexpr (k < kPvMfma) {
        constexpr int u = k / C::kDT, tt = k % C::kDT;
        o[tt] = mfma32(op[k], p_prev.p[u], o[tt]);
      } else {
        constexpr int kk = k - kPvMfma, st = kk / NT, tile = kk % NT;
        s_next.s[tile] = mfma32(op[k], qf[st], st == 0 ? f32x16{} : s_next.s[tile]);
      }
    };
    const float mc = m * c;
    float rs = 0.0f;
    float pe[16 * NT];
    auto valu = [&](auto k_c) {
      constexpr int k = decltype(k_c)::value;
      static_for(std::make_integer_sequence<int, kPerSlot>{}, [&](auto q_c) {
        constexpr int e = k * kPerSlot + decltype(q_c)::value;
        pe[e] = fast_exp2(fmaf(s_cur.s[e >> 4][e & 15], c, -mc));
        if constexpr (e & 1) {
          const uint32_t pk = pack_bf16x2(pe[e - 1], pe[e]);
          p_cur.p[e >> 3][(e >> 1) & 3] = pk;
          rs = dot_sum(pk, rs);
        }
      });
    };
    static_for(std::make_integer_sequence<int, kAhead>{}, [&](auto k_c) { read(k_c); });
    static_for(std::make_integer_sequence<int, kSlots>{}, [&](auto k_c) {
      constexpr int k = decltype(k_c)::value;
      if constexpr (k + kAhead < kSlots) read(std::integral_constant<int, k + kAhead>{});
      mfma(k_c);
      valu(k_c);
      if constexpr (k == kKIssueSlot) issue_k();
      __builtin_amdgcn_sched_barrier(0);
    });
    // keep the first pass ahead of the redo test
#pragma unroll
    for (int u = 0; u < 2 * NT; ++u) asm volatile("" ::"v"(p_cur.p[u]));
    asm volatile("" ::"v"(rs));
    if (wave_ballot(rs > kLazySum) != 0) rs = raise(s_cur, p_cur);
    l += rs;
  };
  // The last iteration, t = nblk - 1 >= 1 (block t may need masking).
  // Its V tile was loaded one iteration ahead into the K slot that no K
  // tile needed any more (kv_c), so the wait at the top covers it.
  auto last = [&](auto kv_c, auto vp, int t, Sc& s_cur, const Pr& p_prev, Pr& p_cur) {
    const int j = __builtin_amdgcn_readfirstlane((int)list[t]);
    wait_vmem<0>();
    barrier_raw();
    pv(vp, p_prev);
    if (needs_mask(j)) mask_block(j, s_cur);
    softmax(s_cur, p_cur);
    pv(kv_c, p_cur);
  };

  if (nblk > 1) {
    // t = 0: no P.V yet
    wait_vmem<0>();
    barrier_raw();
    if (2 < nblk) issue(K0{}, IsK{}, list[2]);
    else issue(K0{}, IsV{}, list[1]);     // nblk = 2: block 1's V into the free K slot
    qk(K1{}, sb);
    const int j0 = __builtin_amdgcn_readfirstlane((int)list[0]);
    if (needs_mask(j0)) mask_block(j0, sa);
    softmax_first(sa, pa);
    int t = 1;
    for (; t + 2 <= nblk - 1; t += 2) {
      steady(K1{}, K0{}, V1{}, V0{}, t, sb, sa, pa, pb);       // t odd
      steady(K0{}, K1{}, V0{}, V1{}, t + 1, sa, sb, pb, pa);   // t + 1 even
    }
    if (t == nblk - 2) {
      steady(K1{}, K0{}, V1{}, V0{}, t, sb, sa, pa, pb);       // t odd
      ++t;
    }
    // t == nblk - 1: its scores are in sb when t is odd, in sa when even
    // block t's V sits in K slot (t + 1) & 1
    if (t & 1) last(K0{}, V0{}, t, sb, pa, pb);
    else last(K1{}, V1{}, t, sa, pb, pa);
  } else if (nblk == 1) {
    const int j = __builtin_amdgcn_readfirstlane((int)list[0]);
    if (needs_mask(j)) mask_block(j, sa);
    softmax_first(sa, pa);
    wait_vmem<0>();
    barrier_raw();
    pv(V0{}, pa);
  }

  // ---- merge the two key halves of each row group, normalise and store ----
  // Wave (rg, kh) finishes O^T tiles kh*kDT/2 .. +kDT/2-1 of its rows; it
  // hands the other half of its tiles to its partner (rg, 1-kh) through the
  // K slots of the ring (free once every wave is past its last P.V, which may
  // read the last block's V tile from a K slot; no load is in flight) and its
  // row max / row sum through `stats`.
  if constexpr (KS == 1) {
    // one wave holds the whole row: normalise and store
    const float lt = sum_with_half_swap(l);
    const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
    if (qrow < Sq && part >= 0) {
      // half of a long row: its normalised fp32 output and (row max, row sum)
      const int64_t pr = (slot * 2 + part) * 64 + 32 * rg + n;
      float* __restrict__ P = a.part_o + pr * D;
#pragma unroll
      for (int t = 0; t < C::kDT; ++t)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d = 32 * t + 8 * g4 + 4 * h;
          *(float4*)(P + d) = float4{o[t][4 * g4 + 0] * inv, o[t][4 * g4 + 1] * inv,
                                     o[t][4 * g4 + 2] * inv, o[t][4 * g4 + 3] * inv};
        }
      if (h == 0) a.part_ml[pr] = float2{m, lt};
    }
    if (part < 0) {   // uniform over the work-group
      // The bf16 output tile is staged in the K slot of the last block (its
      // K tile was read before the last iteration's barrier; nothing reads
      // or loads that slot since) in the K tile's swizzled row layout, then
      // written out as contiguous 16-byte pieces: every wave store covers
      // whole rows of the query block instead of 8 bytes of 32 rows.  The
      // output is not read again here, so the stores are non-temporal.
      unsigned char* const otile = smem + ((max(nblk, 1) - 1) & 1) * C::kTileBytes;
      const int r = 32 * rg + n;
#pragma unroll
      for (int t = 0; t < C::kDT; ++t)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int g = 4 * t + g4;
          *(u32x2*)(otile + r * C::kRowBytes + (g ^ swz_k<D>(r)) * 16 + 8 * (h ^ staged_swap<D>(r))) =
              u32x2{pack_bf16x2(o[t][4 * g4 + 0] * inv, o[t][4 * g4 + 1] * inv),
                    pack_bf16x2(o[t][4 * g4 + 2] * inv, o[t][4 * g4 + 3] * inv)};
        }
      __syncthreads();
      const int rows = min(64, Sq - q0);
      uint16_t* __restrict__ Ot = a.out + q_off + (int64_t)q0 * D;
#pragma unroll
      for (int it = 0; it < 64 * C::G / C::kThreads; ++it) {
        const int e = it * C::kThreads + tid;
        const int rr = e / C::G, g = e % C::G;
        if (rr < rows)
          __builtin_nontemporal_store(staged_row_piece<D>(otile, rr, g),
                                      (u32x4*)(Ot + rr * D + g * 8));
      }
    }
  } else {
  constexpr int kHalf = C::kDT / 2;
  // KH: this wave's key half, as a compile-time value so o[] is indexed statically.
  // The exchange area holds 16-byte pieces: piece (t, g4) of lane l, i.e.
  // elements 4 g4 .. 4 g4 + 3 of the lane's tile t, at ((t * 4 + g4) * 64 + l) * 16.
  auto hand_over = [&](auto kh_c) {
    constexpr int KH = decltype(kh_c)::value;
    unsigned char* xout = smem + w * C::kXchgBytes;
#pragma unroll
    for (int t = 0; t < kHalf; ++t)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x16& src = o[(1 - KH) * kHalf + t];
        *(f32x4*)(xout + ((t * 4 + g4) * kWave + lane) * 16) =
            f32x4{src[4 * g4], src[4 * g4 + 1], src[4 * g4 + 2], src[4 * g4 + 3]};
      }
  };
  __syncthreads();   // the last block's V tile, read from a K slot, is done with
  if (kh == 0) hand_over(std::integral_constant<int, 0>{});
  else hand_over(std::integral_constant<int, 1>{});
  stats[w * 2 * kWave + lane] = m;
  stats[w * 2 * kWave + kWave + lane] = sum_with_half_swap(l);
  __syncthreads();
  const int pw = w ^ 2;   // partner: same rows, other key half
  const unsigned char* xin = smem + pw * C::kXchgBytes;
  const float m_b = stats[pw * 2 * kWave + lane];
  const float l_b = stats[pw * 2 * kWave + kWave + lane];
  const float l_a = sum_with_half_swap(l);
  const float M = fmaxf(m, m_b);   // both finite
  const float al_a = fast_exp2((m - M) * c);
  const float al_b = fast_exp2((m_b - M) * c);
  const float lt = l_a * al_a + l_b * al_b;
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
  const float fa = al_a * inv, fb = al_b * inv;
  // half of a long row: its normalised fp32 output and (row max, row sum)
  const int64_t pr = (slot * 2 + (part < 0 ? 0 : part)) * 64 + 32 * rg + n;
  // The bf16 output tile is staged in V slot 0 (free since the first barrier
  // above) in the K tile's swizzled row layout, then written out by the whole
  // work-group as contiguous 16-byte pieces: the rows of a query block are
  // contiguous in memory, so every wave store covers whole rows instead of
  // 8 bytes of 32 different rows (non-temporal: nothing here reads it again).
  unsigned char* const otile = smem + 2 * C::kTileBytes;
  // The partner's pieces are all read first (one wait for the lot), and the
  // uniform choice of destination is taken once, outside the loops.
  auto finish = [&](auto kh_c) {
    constexpr int KH = decltype(kh_c)::value;
    constexpr int kBase = KH * kHalf;
    f32x4 xb[kHalf][4];
#pragma unroll
    for (int t = 0; t < kHalf; ++t)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        xb[t][g4] = *(const f32x4*)(xin + ((t * 4 + g4) * kWave + lane) * 16);
    auto merged = [&](int t, int g4, int e) {
      return fmaf(o[kBase + t][4 * g4 + e], fa, xb[t][g4][e] * fb);
    };
    if (part >= 0) {
      if (qrow < Sq) {
#pragma unroll
        for (int t = 0; t < kHalf; ++t)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int d = 32 * (kBase + t) + 8 * g4 + 4 * h;
            *(float4*)(a.part_o + pr * D + d) = float4{merged(t, g4, 0), merged(t, g4, 1),
                                                       merged(t, g4, 2), merged(t, g4, 3)};
          }
      }
    } else {
      const int r = 32 * rg + n;
#pragma unroll
      for (int t = 0; t < kHalf; ++t)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int g = 4 * (kBase + t) + g4;   // 16-byte granule of d = 32 (kBase + t) + 8 g4
          *(u32x2*)(otile + r * C::kRowBytes + (g ^ swz_k<D>(r)) * 16 + 8 * (h ^ staged_swap<D>(r))) =
              u32x2{pack_bf16x2(merged(t, g4, 0), merged(t, g4, 1)),
                    pack_bf16x2(merged(t, g4, 2), merged(t, g4, 3))};
        }
    }
  };
  if (part >= 0 && qrow < Sq && kh == 0 && h == 0) a.part_ml[pr] = float2{M, lt};
  if (kh == 0) finish(std::integral_constant<int, 0>{});
  else finish(std::integral_constant<int, 1>{});
  if (part < 0) {   // uniform over the work-group
    __syncthreads();
    const int rows = min(64, Sq - q0);
    uint16_t* __restrict__ Ot = a.out + q_off + (int64_t)q0 * D;
#pragma unroll
    for (int it = 0; it < 64 * C::G / C::kThreads; ++it) {
      const int e = it * C::kThreads + tid;
      const int r = e / C::G, g = e % C::G;
      if (r < rows)
        __builtin_nontemporal_store(staged_row_piece<D>(otile, r, g), (u32x4*)(Ot + r * D + g * 8));
    }
  }
  }

  if constexpr (SRC == kSrcTopk || SRC == kSrcThreshold) {
    if (w == 0 && a.mask_out && !helper) {   // the item writes its row, not its helper
      uint8_t* mo = a.mask_out + ((int64_t)bh * nbk + i) * nbk;
#pragma unroll
      for (int u = 0; u < kMaxKeyChunks; ++u) {
        const int j = 64 * u + lane;
        if (j < nbk) mo[j] = (uint8_t)((selbits[u] >> lane) & 1ull);
      }
    }
  }
}

// Output rows of the long rows split in two: each half left its normalised
// fp32 rows and (row max m, row sum l); the row is their weighted mean with
// weights l * 2^((m - max m) * c), the same log-sum-exp combination the
// split-KV decode's merge uses.  One work-group per 64 slots: every wave reads
// the 64 flags (a slot whose row was not split, flag 0, was written by its
// item), then the work-group merges the flagged slots one after another.
constexpr int kMergeSlots = 64;
template <int D>
__global__ __launch_bounds__(256) void prefill_split_merge_kernel(PrefillArgs a, float c) {
  const int per_bh = a.nbq - a.split_row0;
  const int64_t slots = (int64_t)a.B * a.H * per_bh;
  const int64_t s0 = (int64_t)blockIdx.x * kMergeSlots;
  const int lane = threadIdx.x & 63;
  const bool in = s0 + lane < slots;
  uint64_t todo = wave_ballot(in && a.part_flag[in ? s0 + lane : 0] != 0);
  constexpr int kVec = D / 4;               // float4 per row
  constexpr int kIt = 64 * kVec / 256;      // float4 per thread and half
  while (todo) {
    const int64_t slot = s0 + __ffsll((unsigned long long)todo) - 1;
    todo &= todo - 1;
    const int bh = (int)(slot / per_bh);
    const int i = a.split_row0 + (int)(slot - (int64_t)bh * per_bh);
    // Every load first (rows past Sq read workspace the halves left
    // unwritten, inside the allocation; their results are not stored).
    float4 x0[kIt], x1[kIt];
    float2 m0[kIt], m1[kIt];
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
      const int e = threadIdx.x + 256 * it;
      const int r = e / kVec, d = 4 * (e % kVec);
      const int64_t p0 = slot * 128 + r, p1 = p0 + 64;
      x0[it] = *(const float4*)(a.part_o + p0 * D + d);
      x1[it] = *(const float4*)(a.part_o + p1 * D + d);
      m0[it] = a.part_ml[p0];
      m1[it] = a.part_ml[p1];
    }
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
      const int e = threadIdx.x + 256 * it;
      const int r = e / kVec, d = 4 * (e % kVec);
      const int qrow = 64 * i + r;
      if (qrow < a.Sq) {
        const float mx = fmaxf(m0[it].x, m1[it].x);
        const float w0 = m0[it].y * fast_exp2((m0[it].x - mx) * c);
        const float w1 = m1[it].y * fast_exp2((m1[it].x - mx) * c);
        const float tot = w0 + w1;
        const float inv = tot > 0.0f ? 1.0f / tot : 0.0f;
        const float f0 = w0 * inv, f1 = w1 * inv;
        const float4 u = x0[it], v = x1[it];
        uint16_t* O = a.out + ((int64_t)bh * a.Sq + qrow) * D + d;
        *(u32x2*)O = u32x2{pack_bf16x2(u.x * f0 + v.x * f1, u.y * f0 + v.y * f1),
                           pack_bf16x2(u.z * f0 + v.z * f1, u.w * f0 + v.w * f1)};
      }
    }
  }
}

// Key splits per work item.  At D = 128 always four waves (half the keys
// each): that halves the per-wave registers, so two waves fit per SIMD.  At
// D = 64 the caller chooses (PrefillArgs::ks): two waves over all keys have
// the lowest per-item overhead and win when the items fill the GPU; four waves
// per item put twice the waves on the GPU when items are few (one round of
// resident work-groups or less).
#ifndef BSATTN_KS128
#define BSATTN_KS128 2
#endif

template <int D, int KS, bool CAUSAL, int SRC>
hipError_t launch_t(const PrefillArgs& a, hipStream_t stream) {
  const int BH = a.B * a.H;
  // Item order (item_order.hpp).  Heads per group: as many as one XCD's
  // 4 MB L2 holds the K/V of.  A dense last row (~110 us at B4 H32 S8192
  // D128) outlasts one group's turn, so the last group's rows would trail
  // the launch: at D = 128 the last group's two heaviest rows are issued
  // four groups early (3.5% faster at B1 H32 S16384 D128, 3% at B4 H32
  // S8192 D128, with the L2 hit rate of the plain walk); at D = 64 every
  // group's two heaviest rows go two groups early (6% faster at B4 H32
  // S8192 D64; at D = 128 that measured no faster, since those rows then
  // find their K/V outside the L2 the current group fills).
  int mode = 0, group = 1, lead = 0, ahead = 0, tail = 0;
  if (BH % 8 == 0) {
    mode = 1;
    const int per_xcd = BH / 8;
    const double kv_bytes = 2.0 * a.Sk * D * 2.0;
    int g = (int)(4.0 * 1024 * 1024 / kv_bytes);
    g = max(1, min(g, per_xcd));
    while (per_xcd % g) --g;
    group = g;
    lead = 2;
    ahead = D == 64 ? 2 : 4;
    tail = D == 64 ? 0 : 1;
  }
  const size_t lds = lds_bytes<D, KS>(a.nbk);
  auto kern = prefill_kernel<D, KS, CAUSAL, SRC>;
  if (lds > 64 * 1024) {
    static DeviceHighWater lds_set;   // per instantiation and device
    hipError_t e = lds_set.raise_to((int)lds, [&](int v) {
      return hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, v);
    });
    if (e != hipSuccess) return e;
  }
  // helpers and the merge exist only for the sources that can split
  const int64_t slots =
      (SRC != kSrcList && a.split_min > 0) ? (int64_t)BH * (a.nbq - a.split_row0) : 0;
  const int64_t items = (int64_t)BH * a.nbq + slots;
  // the issue orders of the items and of the long rows' helpers, every
  // quotient they need computed here
  const ItemOrder order = make_item_order(BH, a.nbq, mode, group, lead, ahead, tail != 0);
  const ItemOrder help_order =
      slots > 0 ? make_item_order(BH, a.nbq - a.split_row0, mode, group, 0, 0, false) : ItemOrder{};
  hipLaunchKernelGGL(kern, dim3((unsigned)items), dim3(Cfg<D, KS>::kThreads), lds, stream, a, order,
                     help_order);
  if (slots > 0) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const float c = (float)(1.4426950408889634 / std::sqrt((double)D));
    hipLaunchKernelGGL(prefill_split_merge_kernel<D>,
                       dim3((unsigned)((slots + kMergeSlots - 1) / kMergeSlots)), dim3(256), 0,
                       stream, a, c);
  }
  return hipGetLastError();
}

}  // namespace

size_t prefill_lds_bytes(int D, int nbk) {
  return D == 64 ? std::max(lds_bytes<64, 1>(nbk), lds_bytes<64, 2>(nbk))
                 : lds_bytes<128, BSATTN_KS128>(nbk);
}

template <int D, int KS, bool CAUSAL>
hipError_t launch_src(const PrefillArgs& a, hipStream_t stream) {
  switch (a.src) {
    case kSrcList: return launch_t<D, KS, CAUSAL, kSrcList>(a, stream);
    case kSrcTopk: return launch_t<D, KS, CAUSAL, kSrcTopk>(a, stream);
    case kSrcThreshold: return launch_t<D, KS, CAUSAL, kSrcThreshold>(a, stream);
    default: return launch_t<D, KS, CAUSAL, kSrcMask>(a, stream);
  }
}

template <int D, int KS>
hipError_t launch_ks(const PrefillArgs& a, hipStream_t stream) {
  return a.causal ? launch_src<D, KS, true>(a, stream) : launch_src<D, KS, false>(a, stream);
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  if (a.D == 64) return a.ks == 2 ? launch_ks<64, 2>(a, stream) : launch_ks<64, 1>(a, stream);
  return launch_ks<128, BSATTN_KS128>(a, stream);
}

}  // namespace bsattn
