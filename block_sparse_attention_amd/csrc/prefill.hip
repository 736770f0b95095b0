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
// * 128 threads = 2 wave64s per work item; wave w owns query rows 32w..32w+31.
// * Scores are formed transposed, S^T = K . Q^T, with v_mfma_f32_32x32x16_bf16:
//   the accumulator gives each lane ONE query row (lane % 32) and 32 of the
//   64 keys, so the row max / row sum are in-lane reductions plus a single
//   permlane32 swap, and the exponentiated scores are already laid out as the
//   B operand of O^T = V^T . P^T (no LDS round trip for P).
// * K and V tiles are staged in LDS with a padded row stride; Q^T stays in
//   registers; V^T operands come from ds_read_b64_tr_b16 transposed reads.
// * The next active block's K/V are fetched into registers while the current
//   block is computed.
// * The mask row is compacted on the fly: a 64-column ballot per step gives
//   the ascending list of selected key blocks, consumed bit by bit.
// * Work items are issued heaviest-first (last query block first), and when
//   batch*heads is a multiple of 8 each head's items stay on one XCD so its
//   K/V stay in that XCD's L2.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace bsattn {

namespace {

constexpr int kThreads = 128;
constexpr float kLazy = 8.0f;   // log2 headroom before the running max must move

template <int D>
struct Cfg {
  static constexpr int kStride = D + 16;              // LDS row stride (bf16 elements)
  static constexpr int kRowChunks = D / 8;            // 16-byte chunks per row
  static constexpr int kPerThread = 64 * kRowChunks / kThreads;
  static constexpr int kSteps = D / 16;               // k-steps of S^T = K . Q^T
  static constexpr int kDT = D / 32;                  // 32-row tiles of O^T
};

// Active key blocks of one query-block row, read from the mask row.
struct MaskRowIter {
  const uint8_t* row;
  int lim;
  int c0;
  uint64_t bits;
  __device__ __forceinline__ void init(const uint8_t* r, int l) {
    row = r;
    lim = l;
    c0 = -kWave;
    bits = 0;
  }
  __device__ __forceinline__ int next() {
    while (bits == 0) {
      c0 += kWave;
      if (c0 >= lim) return -1;
      const int j = c0 + lane_id();
      bits = wave_ballot(j < lim && row[j] != 0);
    }
    const int t = __builtin_ctzll(bits);
    bits &= bits - 1;
    return c0 + t;
  }
};

// Active key blocks of one row, read from a precomputed list.
struct ListIter {
  const int32_t* list;
  int n;
  int pos;
  int lim;
  __device__ __forceinline__ void init(const int32_t* l, int count, int lim_) {
    list = l;
    n = count;
    pos = 0;
    lim = lim_;
  }
  __device__ __forceinline__ int next() {
    while (pos < n) {
      const int j = __builtin_amdgcn_readfirstlane(list[pos]);
      ++pos;
      if (j >= 0 && j < lim) return j;
    }
    return -1;
  }
};

// Work item L -> (batch*head, query block).  Query blocks are issued last
// first.  In mode 1 (batch*heads divisible by 8) item L runs on XCD L % 8;
// the XCD owns heads xcd, xcd+8, ...; it walks them in groups of `group`
// heads, query blocks descending, heads interleaved within a group.
__device__ __forceinline__ void map_item(int L, int BH, int nb, int mode, int group, int& bh,
                                         int& i) {
  if (mode == 1) {
    const int xcd = L & 7;
    const int k = L >> 3;
    const int per = group * nb;
    const int grp = k / per;
    const int r = k - grp * per;
    const int ii = r / group;
    const int hh = grp * group + (r - ii * group);
    i = nb - 1 - ii;
    bh = xcd + 8 * hh;
  } else {
    const int ii = L / BH;
    bh = L - ii * BH;
    i = nb - 1 - ii;
  }
}

__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* p) {
  bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((BSATTN_LDS bf16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

template <int D, bool CAUSAL, bool LIST>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void
prefill_kernel(PrefillArgs a, int map_mode, int group) {
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[64 * C::kStride];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[64 * C::kStride];

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int h = lane >> 5;   // which half of the key rows / k-group this lane holds
  const int n = lane & 31;   // query row within the wave

  const int nb = a.nb;
  const int S = a.S;
  int bh, i;
  map_item(blockIdx.x, a.B * a.H, nb, map_mode, group, bh, i);

  const int64_t head_off = (int64_t)bh * S * D;
  const uint16_t* __restrict__ Q = a.q + head_off;
  const uint16_t* __restrict__ K = a.k + head_off;
  const uint16_t* __restrict__ V = a.v + head_off;
  const int q0 = i * 64;
  const int qrow = q0 + 32 * w + n;

  // Q^T as the B operand of S^T = K . Q^T: lane holds row qrow, dims 16s + 8h .. +8.
  u32x4 qf[C::kSteps];
#pragma unroll
  for (int s = 0; s < C::kSteps; ++s) {
    if (qrow < S)
      qf[s] = *(const u32x4*)(Q + (int64_t)qrow * D + 16 * s + 8 * h);
    else
      qf[s] = u32x4{0, 0, 0, 0};
  }

  f32x16 o[C::kDT];
#pragma unroll
  for (int t = 0; t < C::kDT; ++t) o[t] = f32x16{};
  float m = -INFINITY;
  float l = 0.0f;
  const float c = (float)(1.4426950408889634 / __builtin_sqrt((double)D));

  const int lim = CAUSAL ? min(i + 1, nb) : nb;
  MaskRowIter mit;
  ListIter lit;
  if constexpr (LIST) {
    const int64_t row = (int64_t)bh * nb + i;
    int count = a.cnt[row];
    count = max(0, min(count, nb));
    lit.init(a.idx + row * nb, count, lim);
  } else {
    mit.init(a.mask + ((int64_t)bh * nb + i) * nb, lim);
  }
  auto next_block = [&]() -> int {
    if constexpr (LIST) return lit.next();
    else return mit.next();
  };

  u32x4 kr[C::kPerThread], vr[C::kPerThread];
  // Rows past the end of the sequence read the last row instead (always in
  // bounds); their scores are masked to -inf and, for V, zeroed, so the values
  // never matter except that they must be finite.
  auto fetch = [&](int j) {
#pragma unroll
    for (int t = 0; t < C::kPerThread; ++t) {
      const int chunk = tid + kThreads * t;
      const int key = min(j * 64 + chunk / C::kRowChunks, S - 1);
      const int64_t off = (int64_t)key * D + (chunk % C::kRowChunks) * 8;
      kr[t] = *(const u32x4*)(K + off);
      vr[t] = *(const u32x4*)(V + off);
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int t = 0; t < C::kPerThread; ++t) {
      const int chunk = tid + kThreads * t;
      const int r = chunk / C::kRowChunks;
      const int c8 = chunk % C::kRowChunks;
      *(u32x4*)(Ks + r * C::kStride + c8 * 8) = kr[t];
      *(u32x4*)(Vs + r * C::kStride + c8 * 8) = vr[t];
    }
  };

  // lane coordinates for the transposed V reads
  const int tr_r = (lane >> 2) & 3;
  const int tr_m = lane & 3;
  const int tr_g = (lane >> 4) & 1;

  int j = next_block();
  if (j >= 0) fetch(j);
  while (j >= 0) {
    __syncthreads();  // every wave is done with the previous tile
    stage();
    __syncthreads();
    const int jn = next_block();
    if (jn >= 0) fetch(jn);  // in flight while this block is computed

    // ---- S^T = K . Q^T : two 32-key tiles ----
    f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
    for (int st = 0; st < C::kSteps; ++st) {
      const u32x4 a0 = *(const u32x4*)(Ks + n * C::kStride + 16 * st + 8 * h);
      const u32x4 a1 = *(const u32x4*)(Ks + (32 + n) * C::kStride + 16 * st + 8 * h);
      s0 = mfma32(a0, qf[st], s0);
      s1 = mfma32(a1, qf[st], s1);
    }

    // ---- causal diagonal block and ragged tail ----
    const int kbase = j * 64;
    if ((CAUSAL && j == i) || kbase + 64 > S) {
      // keys of this block at or beyond `vis` are hidden from this lane's query row
      int vis = S - kbase;
      if (CAUSAL && j == i) vis = min(vis, qrow - kbase + 1);
#pragma unroll
      for (int ii = 0; ii < 16; ++ii) {
        const int k0 = 8 * (ii >> 2) + 4 * h + (ii & 3);
        if (k0 >= vis) s0[ii] = -INFINITY;
        if (k0 + 32 >= vis) s1[ii] = -INFINITY;
      }
    }

    // ---- online softmax (base 2) ----
    // The running maximum m only serves as the exponent offset, so it is
    // raised lazily: only when some row's block maximum exceeds it by more
    // than kLazy (in log2 units) is m moved and o, l rescaled.  Until then
    // probabilities may reach 2^kLazy, harmless in fp32 and bf16.
    float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
    for (int ii = 1; ii < 16; ++ii) mx = fmaxf(mx, fmaxf(s0[ii], s1[ii]));
    mx = max_with_half_swap(mx);
    if (wave_ballot((mx - m) * c > kLazy) != 0) {
      const float m_new = fmaxf(m, mx);
      const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
      const float alpha = fast_exp2((m - m_use) * c);
      l *= alpha;
#pragma unroll
      for (int t = 0; t < C::kDT; ++t)
#pragma unroll
        for (int ii = 0; ii < 16; ++ii) o[t][ii] *= alpha;
      m = m_new;
    }
    const float mc = (m == -INFINITY) ? 0.0f : m * c;
    float rs = 0.0f;
#pragma unroll
    for (int ii = 0; ii < 16; ++ii) {
      s0[ii] = fast_exp2(fmaf(s0[ii], c, -mc));
      s1[ii] = fast_exp2(fmaf(s1[ii], c, -mc));
      rs += s0[ii] + s1[ii];
    }
    l += rs;

    // ---- O^T += V^T . P^T : four 16-key steps ----
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const f32x16& sp = (u < 2) ? s0 : s1;
      const int base = 8 * (u & 1);
      const u32x4 pb = u32x4{pack_bf16x2(sp[base + 0], sp[base + 1]),
                             pack_bf16x2(sp[base + 2], sp[base + 3]),
                             pack_bf16x2(sp[base + 4], sp[base + 5]),
                             pack_bf16x2(sp[base + 6], sp[base + 7])};
      const int row0 = 16 * u + 4 * h + tr_r;
#pragma unroll
      for (int t = 0; t < C::kDT; ++t) {
        const int col = 32 * t + 16 * tr_g + 4 * tr_m;
        const u32x2 lo = lds_read_tr16(Vs + row0 * C::kStride + col);
        const u32x2 hi = lds_read_tr16(Vs + (row0 + 8) * C::kStride + col);
        o[t] = mfma32(u32x4{lo[0], lo[1], hi[0], hi[1]}, pb, o[t]);
      }
    }
    j = jn;
  }

  // ---- normalise and store ----
  const float lt = sum_with_half_swap(l);
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
  if (qrow < S) {
    uint16_t* __restrict__ O = a.out + head_off + (int64_t)qrow * D;
#pragma unroll
    for (int t = 0; t < C::kDT; ++t)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * t + 8 * g4 + 4 * h;
        const u32x2 val = u32x2{pack_bf16x2(o[t][4 * g4 + 0] * inv, o[t][4 * g4 + 1] * inv),
                                pack_bf16x2(o[t][4 * g4 + 2] * inv, o[t][4 * g4 + 3] * inv)};
        *(u32x2*)(O + d) = val;
      }
  }
}

template <int D, bool CAUSAL, bool LIST>
hipError_t launch_t(const PrefillArgs& a, hipStream_t stream) {
  const int BH = a.B * a.H;
  int mode = 0, group = 1;
  if (BH % 8 == 0) {
    mode = 1;
    const int per_xcd = BH / 8;
    const double kv_bytes = 2.0 * a.S * D * 2.0;
    int g = (int)(4.0 * 1024 * 1024 / kv_bytes);
    g = max(1, min(g, per_xcd));
    while (per_xcd % g) --g;
    group = g;
  }
  const int64_t items = (int64_t)BH * a.nb;
  hipLaunchKernelGGL((prefill_kernel<D, CAUSAL, LIST>), dim3((unsigned)items), dim3(kThreads), 0,
                     stream, a, mode, group);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  const bool list = a.mask == nullptr;
  if (a.D == 64) {
    if (a.causal) return list ? launch_t<64, true, true>(a, stream) : launch_t<64, true, false>(a, stream);
    return list ? launch_t<64, false, true>(a, stream) : launch_t<64, false, false>(a, stream);
  }
  if (a.causal) return list ? launch_t<128, true, true>(a, stream) : launch_t<128, true, false>(a, stream);
  return list ? launch_t<128, false, true>(a, stream) : launch_t<128, false, false>(a, stream);
}

}  // namespace bsattn
