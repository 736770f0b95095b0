// Split-KV sparse GQA decode for gfx950 (one query token per sequence).
//
// What is computed follows the TileLang block-sparse Flash-Attention guide,
// §6–§6.2: for each (batch, KV head) the list of selected 64-token blocks is
// cut into num_splits contiguous ranges (the first slots % splits ranges one
// slot longer); padded (-1) and out-of-range entries are skipped; keys at or
// beyond the sequence length are masked; each range produces a normalised
// partial output and its base-2 log-sum-exp, and a merge kernel combines the
// ranges with weights 2^(lse - max lse) (§6.1).  Query head hq reads KV head
// hq / (Hq / Hkv); up to 64 query heads share a KV head (§6.1: valid_block_H =
// min(64, group)).  V's head dim may differ from K's (§9.2: dim and dim_v).
//
// CDNA4 mapping (not the guide's kernel design):
// * one work-group of 4 wave64s per (batch, KV head, split, 16-head column
//   tile); the waves take the range's slots round-robin and are combined
//   through LDS at the end;
// * per 64-token block, S^T = K . Q^T on v_mfma_f32_16x16x32_bf16 with 16 of
//   the group's query heads as the columns (K rows loaded straight from HBM
//   into the A-operand layout, 16 bytes per lane); groups of more than 16
//   heads take one work-group per 16-head tile, whose K/V reads of the same
//   blocks meet in the caches;
// * the exponentiated scores are already the B operand of O^T = V^T . P^T;
//   V goes through LDS, read transposed with ds_read_b64_tr_b16;
// * software pipeline per wave: the next selected block's K loads are issued
//   right after the current block's S^T, its V loads right after the current
//   block's P.V, so a block's loads are in flight during the previous block's
//   softmax and P.V.  Loads go through a buffer resource bounded to the
//   block's valid rows, so rows past the sequence end read as zero (no
//   branches around loads); their scores are masked.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace bsattn {

namespace {

// Waves per work-group: four (one per SIMD) measured 2-5% faster per call than
// eight on the 8-batch, 8-KV-head, 4-split decode: the split's blocks spread
// over fewer waves, each keeping more blocks in its load pipeline.
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;

__device__ __forceinline__ f32x4 mfma16(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* p) {
  bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((BSATTN_LDS bf16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Buffer resource over one 64-token block of one KV head: loads at byte
// offsets past `bytes` return zero instead of touching memory, which is how
// rows past the sequence end are kept out of the block.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const uint16_t* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, 0x00020000);
}
// voff is range-checked against the resource; soff is a small constant
// added on top (kept within the row that voff addresses).
__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4,
                            __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}

template <bool B>
struct BoolC {
  static constexpr bool value = B;
};

// D: key/query head dim; DV: value (and output) head dim.
template <int D, int DV>
struct DCfg {
  static constexpr int kStride = DV + 16;    // LDS row stride of a V half tile
  static constexpr int kSteps = D / 32;      // k-steps of S^T = K . Q^T
  static constexpr int kDT = DV / 16;        // 16-row tiles of O^T
  static constexpr int kRowChunks = DV / 8;  // 16-byte chunks per V token row
  static constexpr int kVPer = 64 * kRowChunks / kWave;  // V chunks per lane per block
  static constexpr int kTokPerInstr = kWave / kRowChunks;  // V tokens per load instruction
  // bf16 elements per wave: the V half tile, or the combine's floats
  // (16 m, 16 l, 16 x DV o), whichever is larger
  static constexpr int kWaveLds =
      32 * kStride > (32 + 16 * DV) * 2 ? 32 * kStride : (32 + 16 * DV) * 2;
};

template <int D>
struct KTile {
  u32x4 f[4][D / 32];
};
template <int D, int DV>
struct VTile {
  u32x4 f[DCfg<D, DV>::kVPer];
};

// Position of the r-th (from 0) set bit of x; x has more than r set bits.
__device__ __forceinline__ int nth_set_bit(uint64_t x, int r) {
  int pos = 0;
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) {
    const int c = __popcll(x & ((1ull << w) - 1));
    if (r >= c) {
      r -= c;
      x >>= w;
      pos += w;
    }
  }
  return pos;
}

// A selected block: its index in the sequence, and for the paged cache its physical page.
struct BlockRef {
  int blk;
  int page;
};

template <int D, int DV, int MODE>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(DecodeArgs a, int final_out) {
  using C = DCfg<D, DV>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[kWaves * C::kWaveLds];

  const int sid = blockIdx.x;
  const int G = a.Hq / a.Hkv;
  const int nct = (G + 15) / 16;                      // 16-head column tiles per KV head
  const int kvh = (int)blockIdx.y / nct;
  const int col0 = 16 * ((int)blockIdx.y - kvh * nct);  // first group head of this tile
  const int Gt = min(16, G - col0);                   // heads in this tile
  const int b = blockIdx.z;
  const int ns = a.num_splits;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int col = lane & 15;     // query column of the 16x16 tiles
  const int grp = lane >> 4;     // k-group / row group
  uint16_t* Vs = lds + w * C::kWaveLds;

  // sequence extent; a malformed range (or a negative paged length) is treated as empty
  int start = 0, len = 0;
  if constexpr (MODE == kDecodePaged) {
    len = max(a.cache_seqlens[b], 0);
  } else {
    start = a.cu_seqlens[b];
    const int end = a.cu_seqlens[b + 1];
    len = (end >= start && end <= a.total_k && start >= 0) ? end - start : 0;
  }
  const int nbb = (len + 63) / 64;
  const int ratio = MODE == kDecodePaged ? a.page_size / 64 : 1;   // 64-token blocks per page

  const int nslots = a.max_sel;
  const int64_t sel_row = ((int64_t)b * a.Hkv + kvh) * nslots;

  // Index forms: this split takes a contiguous range of the (compact, -1
  // padded) list, and wave w its slots my_start + w + kWaves j.
  // Mask form: the row's selected blocks are ranked by column; this split
  // takes ranks my_start .. my_start + my_len - 1 and wave w ranks
  // my_start + w + kWaves j, so every split and every wave gets an even share
  // of the selected blocks wherever they sit in the row.  The row's
  // selection is read kMaskBatch columns at a time as lane-uniform words.
  constexpr int kMaskWords = 8;
  constexpr int kMaskBatch = kMaskWords * kWave;
  uint64_t mw[kMaskWords] = {};
  auto mask_words = [&](int q0) {
    uint8_t mb[kMaskWords];
#pragma unroll
    for (int u = 0; u < kMaskWords; ++u)   // unconditional, clamped: all loads in flight at once
      mb[u] = a.block_mask[sel_row + min(q0 + kWave * u + lane, nslots - 1)];
#pragma unroll
    for (int u = 0; u < kMaskWords; ++u) {
      const int j = q0 + kWave * u + lane;
      mw[u] = wave_ballot(j < nslots && j < nbb && mb[u] != 0);
    }
  };
  int my_len, my_start;
  if constexpr (MODE == kDecodeMask) {
    int nsel = 0;
    for (int q0 = 0; q0 < nslots; q0 += kMaskBatch) {
      mask_words(q0);
#pragma unroll
      for (int u = 0; u < kMaskWords; ++u) nsel += __popcll(mw[u]);
    }
    const int per = nsel / ns, extra = nsel % ns;
    my_len = per + (sid < extra ? 1 : 0);
    my_start = per * sid + min(sid, extra);
  } else {
    const int bps = nslots / ns, rem = nslots % ns;
    my_len = bps + (sid < rem ? 1 : 0);
    my_start = bps * sid + min(sid, rem);
  }
  const int nper = my_len > w ? (my_len - w + kWaves - 1) / kWaves : 0;

  const uint32_t rsb = (uint32_t)a.Hkv * D * 2;    // bytes between consecutive K tokens
  const uint32_t rsbv = (uint32_t)a.Hkv * DV * 2;  // bytes between consecutive V tokens
  const float c = (float)(1.4426950408889634 / __builtin_sqrt((double)D));

  // Q^T as the B operand: column col = query head kvh*G + col0 + col (zero when col >= Gt).
  u32x4 qf[C::kSteps];
  {
    const int hq = kvh * G + col0 + col;
#pragma unroll
    for (int s = 0; s < C::kSteps; ++s) {
      if (col < Gt)
        qf[s] = *(const u32x4*)(a.q + ((int64_t)b * a.Hq + hq) * D + 32 * s + 8 * grp);
      else
        qf[s] = u32x4{0, 0, 0, 0};
    }
  }

  f32x4 o[C::kDT];
#pragma unroll
  for (int t = 0; t < C::kDT; ++t) o[t] = f32x4{};
  float m = -INFINITY;
  float l = 0.0f;

  const int tr_r = (lane >> 2) & 3;
  const int tr_m = lane & 3;

  // per-lane byte offsets inside a block: K rows 16*tt + col, k-chunks
  // 32*s + 8*grp (A-operand layout); V chunk lane + 64*t = (token, 16 bytes)
  uint32_t koff[4];
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) koff[tt] = (uint32_t)(16 * tt + col) * rsb + 16u * grp;
  const uint32_t voff0 = (uint32_t)(lane / C::kRowChunks) * rsbv + 16u * (lane % C::kRowChunks);
  const uint32_t vstep = (uint32_t)C::kTokPerInstr * rsbv;

  // first row of a block: packed, row start + 64 blk; paged, row (blk % ratio) * 64 of its page
  // (tokens rs bytes apart, rows of hd elements)
  auto rsrc = [&](const uint16_t* p, BlockRef ref, uint32_t rs, int hd) {
    const int ntok = min(64, len - ref.blk * 64);
    const int64_t row = MODE == kDecodePaged
                            ? (int64_t)ref.page * a.page_size + (int64_t)(ref.blk % ratio) * 64
                            : (int64_t)start + (int64_t)ref.blk * 64;
    const uint16_t* base = p + row * (rs / 2) + (int64_t)kvh * hd;
    return block_rsrc(base, (uint32_t)(ntok - 1) * rs + hd * 2);
  };
  auto load_k = [&](BlockRef blk, KTile<D>& kt) {
    const __amdgpu_buffer_rsrc_t r = rsrc(a.k, blk, rsb, D);
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int s = 0; s < C::kSteps; ++s) kt.f[tt][s] = bload16(r, koff[tt], 64u * s);
  };
  auto load_v = [&](BlockRef blk, VTile<D, DV>& vt) {
    const __amdgpu_buffer_rsrc_t r = rsrc(a.v, blk, rsbv, DV);
    // recomputed per block (not hoisted): one offset register instead of kVPer
    uint32_t vo = voff0;
    asm volatile("" : "+v"(vo));
#pragma unroll
    for (int t = 0; t < C::kVPer; ++t) vt.f[t] = bload16(r, vo + vstep * t, 0);
  };

  // one selected block: S^T, softmax, O^T += V^T . P^T; with MORE, the next
  // block's K loads go out after S^T and its V loads after P.V
  auto process = [&](BlockRef blk, BlockRef nblk, KTile<D>& kt, VTile<D, DV>& vt, auto more_c) {
    constexpr bool kMore = decltype(more_c)::value;
    const int ntok = min(64, len - blk.blk * 64);
    // S^T tiles: token 16*tt + 4*grp + r, query column col
    f32x4 sc[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      sc[tt] = f32x4{};
#pragma unroll
      for (int s = 0; s < C::kSteps; ++s) sc[tt] = mfma16(kt.f[tt][s], qf[s], sc[tt]);
    }
    if constexpr (kMore) load_k(nblk, kt);
    if (ntok < 64) {
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (16 * tt + 4 * grp + r >= ntok) sc[tt][r] = -INFINITY;
    }

    float mx = sc[0][0];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sc[tt][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m, mx);
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = fast_exp2((m - m_use) * c);
    const float mc = m_use * c;
    float rs = 0.0f;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sc[tt][r] = fast_exp2(fmaf(sc[tt][r], c, -mc));
        rs += sc[tt][r];
      }
    l = l * alpha + rs;
    m = m_new;
    // P^T as the B operand of the two 32-token halves
    u32x4 pb[2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
      pb[u] = u32x4{pack_bf16x2(sc[2 * u][0], sc[2 * u][1]),
                    pack_bf16x2(sc[2 * u][2], sc[2 * u][3]),
                    pack_bf16x2(sc[2 * u + 1][0], sc[2 * u + 1][1]),
                    pack_bf16x2(sc[2 * u + 1][2], sc[2 * u + 1][3])};
#pragma unroll
    for (int t = 0; t < C::kDT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) o[t][r] *= alpha;

    // O^T += V^T . P^T in two 32-token halves, each staged through LDS
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      wave_lds_sync();  // previous reads of this wave's buffer are done
#pragma unroll
      for (int t = 0; t < C::kVPer / 2; ++t) {
        const int chunk = lane + kWave * (t + u * (C::kVPer / 2));
        const int tok = chunk / C::kRowChunks - 32 * u;
        const int c8 = chunk % C::kRowChunks;
        *(u32x4*)(Vs + tok * C::kStride + c8 * 8) = vt.f[t + u * (C::kVPer / 2)];
      }
      wave_lds_sync();
      const int row0 = 4 * grp + tr_r;
#pragma unroll
      for (int t = 0; t < C::kDT; ++t) {
        const int cc = 16 * t + 4 * tr_m;
        const u32x2 lo = lds_read_tr16(Vs + row0 * C::kStride + cc);
        const u32x2 hi = lds_read_tr16(Vs + (row0 + 16) * C::kStride + cc);
        o[t] = mfma16(u32x4{lo[0], lo[1], hi[0], hi[1]}, pb[u], o[t]);
      }
    }
    if constexpr (kMore) load_v(nblk, vt);
  };

  for (int c0 = 0; c0 < nper; c0 += kWave) {
    // this wave's next 64 slots: lane j holds slot (index forms) or rank
    // (mask form) my_start + w + kWaves * (c0 + j)
    int bv = -1;
    const bool want = c0 + lane < nper;
    const int slot = my_start + w + kWaves * (c0 + lane);
    if constexpr (MODE == kDecodeMask) {
      // the column of rank `slot`: walk the row's words, counting selections
      int seen = 0;
      for (int q0 = 0; q0 < nslots; q0 += kMaskBatch) {
        if (nslots > kMaskBatch) mask_words(q0);   // one batch stays from the count
#pragma unroll
        for (int u = 0; u < kMaskWords; ++u) {
          const int pc = __popcll(mw[u]);
          const int r = slot - seen;
          if (want && r >= 0 && r < pc) bv = q0 + kWave * u + nth_set_bit(mw[u], r);
          seen += pc;
        }
      }
    } else if (want) {
      bv = a.block_indices[sel_row + slot];
    }
    bool ok = bv >= 0 && bv < nbb;
    int pg = 0;
    if constexpr (MODE == kDecodePaged) {
      // logical page -> physical page; entries outside the table or the cache select nothing
      const int lp = ok ? bv / ratio : 0;
      ok = ok && lp < a.max_blocks_per_seq;
      pg = ok ? a.block_table[(int64_t)b * a.max_blocks_per_seq + lp] : -1;
      ok = ok && pg >= 0 && pg < a.num_pages;
    }
    uint64_t vm = wave_ballot(ok);
    const int n = __builtin_popcountll(vm);
    if (n == 0) continue;
    auto take = [&]() {
      const int j = __builtin_ctzll(vm);
      vm &= vm - 1;
      return BlockRef{__builtin_amdgcn_readlane(bv, j), __builtin_amdgcn_readlane(pg, j)};
    };
    KTile<D> kt;
    VTile<D, DV> vt;
    BlockRef blk = take();
    load_k(blk, kt);
    load_v(blk, vt);
    for (int i = 1; i < n; ++i) {
      const BlockRef nblk = take();
      process(blk, nblk, kt, vt, BoolC<true>{});
      blk = nblk;
    }
    process(blk, BlockRef{0, 0}, kt, vt, BoolC<false>{});
  }

  // ---- combine the waves of this split ----
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  wave_lds_sync();
  __syncthreads();
  float* red = (float*)(lds + w * C::kWaveLds);   // [16 m][16 l][16 * DV o]
  if (grp == 0) {
    red[col] = m;
    red[16 + col] = l;
  }
#pragma unroll
  for (int t = 0; t < C::kDT; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[32 + col * DV + 16 * t + 4 * grp + r] = o[t][r];
  __syncthreads();

  for (int e = tid; e < Gt * DV; e += kThreads) {
    const int qn = e / DV;
    const int d = e - qn * DV;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, ((float*)(lds + ww * C::kWaveLds))[qn]);
    float L = 0.0f, acc = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) {
        const float* rw = (const float*)(lds + ww * C::kWaveLds);
        const float mw = rw[qn];
        const float wt = (mw == -INFINITY) ? 0.0f : fast_exp2((mw - M) * c);
        L += rw[16 + qn] * wt;
        acc += rw[32 + qn * DV + d] * wt;
      }
    }
    const float val = L > 0.0f ? acc / L : 0.0f;
    const int hq = kvh * G + col0 + qn;
    if (final_out) {
      a.out[((int64_t)b * a.Hq + hq) * DV + d] = float_to_bf16_bits(val);
    } else {
      const int64_t pi = ((int64_t)b * a.Hq + hq) * ns + sid;
      a.o_part[pi * DV + d] = val;
      if (d == 0) a.lse[pi] = L > 0.0f ? M * c + __log2f(L) : -INFINITY;
    }
  }
}

// One work-group per (batch, query head): weights 2^(lse_s - max lse),
// accumulated in one pass with a running maximum so the loads of all splits
// are independent of each other.
template <int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(DecodeArgs a) {
  const int64_t bq = blockIdx.x;
  const int ns = a.num_splits;
  const int d = threadIdx.x;
  const float* lse = a.lse + bq * ns;
  const float* op = a.o_part + bq * ns * D;
  float M = -INFINITY, num = 0.0f, den = 0.0f;
#pragma unroll 4
  for (int s = 0; s < ns; ++s) {
    const float ls = lse[s];
    const float x = op[(int64_t)s * D + d];
    if (ls == -INFINITY) continue;
    if (ls > M) {
      const float sc = (M == -INFINITY) ? 0.0f : fast_exp2(M - ls);
      num *= sc;
      den *= sc;
      M = ls;
    }
    const float wt = fast_exp2(ls - M);
    den += wt;
    num += wt * x;
  }
  a.out[bq * D + d] = float_to_bf16_bits(den > 0.0f ? num / den : 0.0f);
}

template <int D, int DV, int MODE>
hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
  const int final_out = a.num_splits == 1 ? 1 : 0;
  const int nct = (a.Hq / a.Hkv + 15) / 16;
  hipLaunchKernelGGL((decode_split_kernel<D, DV, MODE>), dim3(a.num_splits, a.Hkv * nct, a.B),
                     dim3(kThreads), 0, stream, a, final_out);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || final_out) return e;
  hipLaunchKernelGGL(decode_merge_kernel<DV>, dim3((unsigned)((int64_t)a.B * a.Hq)), dim3(DV), 0,
                     stream, a);
  return hipGetLastError();
}


template <int MODE>
hipError_t launch_mode(const DecodeArgs& a, hipStream_t stream) {
  if (a.D == 64) return a.Dv == 64 ? launch_t<64, 64, MODE>(a, stream) : launch_t<64, 128, MODE>(a, stream);
  return a.Dv == 64 ? launch_t<128, 64, MODE>(a, stream) : launch_t<128, 128, MODE>(a, stream);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  if (a.mode == kDecodeMask) return launch_mode<kDecodeMask>(a, stream);
  if (a.mode == kDecodePaged) return launch_mode<kDecodePaged>(a, stream);
  return launch_mode<kDecodeIndices>(a, stream);
}

}  // namespace bsattn
