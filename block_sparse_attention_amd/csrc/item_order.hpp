// Issue order of the forward's work items: work item L (the work-group's
// index) -> (batch * head, query block).  Host-compilable, so the order can
// be checked on the CPU as a bijection.
//
// Query blocks are issued last first: under a causal mask the last query
// blocks see the most key blocks, so the heaviest items start first and the
// light ones fill the end of the launch.
//
// Mode 0: query-block-major over all batch*heads.
//
// Mode 1 (batch*heads divisible by 8): item L runs on XCD L % 8, which owns
// heads xcd, xcd + 8, ...  The XCD walks its heads in groups of `group`
// (heads interleaved within a group, query blocks descending), so the K/V of
// the heads in flight stay in that XCD's L2.  A look-ahead (lead > 0,
// ahead > 0) issues the first `lead` query blocks of some groups early, so a
// row much heavier than a group's time slice (a dense last row) does not
// start only when its group's turn comes and hold up the end of the launch:
//  * tail = false: those of group j + ahead just before the rest of group j
//    (and those of groups 0 .. ahead-1 first);
//  * tail = true: only those of the last group, just before group
//    n - 1 - ahead (n groups per XCD; ahead is clamped to n - 1), every other
//    group walking in plain order.
// lead = 0 or ahead = 0 gives the plain group walk.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define BSATTN_HD __host__ __device__ __forceinline__
#else
#define BSATTN_HD inline
#endif

namespace bsattn {

// Division by a divisor fixed at launch, for dividends in [0, 2^31): with
// l = ceil(log2 d) and m = ceil(2^(31 + l) / d) (below 2^32), x / d equals
// (x * m) >> (31 + l): m * d exceeds 2^(31 + l) by less than d, so the
// product's excess over x / d * 2^(31 + l) stays below x * d / 2^(31 + l) < 1
// quotient step.  Two scalar multiplies and a shift on the device instead
// of a float reciprocal and a correction sequence.
struct FastDiv {
  uint32_t m;
  int sh;
};
BSATTN_HD FastDiv make_fastdiv(uint32_t d) {
  FastDiv f{0u, 0};
  if (d == 0) return f;   // never divided by (guarded by the callers)
  int l = 0;
  while ((1ull << l) < d) ++l;
  const unsigned long long num = 1ull << (31 + l);
  f.m = (uint32_t)((num + d - 1) / d);
  f.sh = 31 + l;
  return f;
}
BSATTN_HD int fdiv(int x, const FastDiv& f) {
  return (int)(((unsigned long long)(uint32_t)x * f.m) >> f.sh);
}

// The issue order of one launch, with every quotient the mapping needs
// precomputed on the host.
struct ItemOrder {
  int mode, BH, nb, group, lead, ahead, tail;
  int n, heavy_n, light_n, per, a0, full;   // mode 1
  FastDiv div_per, div_group, div_light, div_heavy, div_bh;
};

BSATTN_HD ItemOrder make_item_order(int BH, int nb, int mode, int group, int lead, int ahead,
                                    bool tail) {
  ItemOrder o{};
  o.mode = mode;
  o.BH = BH;
  o.nb = nb;
  o.div_bh = make_fastdiv((uint32_t)BH);
  if (mode != 1) return o;
  const int n = (BH / 8) / group;   // groups on each XCD
  if (lead > nb) lead = nb;
  if (ahead > (tail ? n - 1 : n)) ahead = tail ? n - 1 : n;
  if (lead <= 0 || ahead <= 0) {
    lead = 0;
    ahead = 0;
  }
  o.group = group;
  o.lead = lead;
  o.ahead = ahead;
  o.tail = tail ? 1 : 0;
  o.n = n;
  o.heavy_n = lead * group;          // look-ahead items per group
  o.light_n = (nb - lead) * group;   // the rest of a group
  o.per = o.heavy_n + o.light_n;
  o.a0 = (n - 1 - ahead) * o.per;
  o.full = (n - ahead) * o.per;
  o.div_per = make_fastdiv((uint32_t)o.per);
  o.div_group = make_fastdiv((uint32_t)group);
  o.div_light = make_fastdiv((uint32_t)o.light_n);
  o.div_heavy = make_fastdiv((uint32_t)o.heavy_n);
  return o;
}

BSATTN_HD void map_item(const ItemOrder& o, int L, int& bh, int& i) {
  if (o.mode == 1) {
    const int xcd = L & 7;
    const int k = L >> 3;
    const int group = o.group, lead = o.lead, ahead = o.ahead, n = o.n;
    const int heavy_n = o.heavy_n, light_n = o.light_n, per = o.per;
    int grp, ii, hin;
    if (o.tail) {
      // groups 0 .. n-2-ahead | heavy of group n-1 | groups n-1-ahead .. n-2 | light of group n-1
      const int a0 = o.a0;
      int r;
      if (ahead == 0 || k < a0) {
        grp = fdiv(k, o.div_per);
        r = k - grp * per;
      } else if (k < a0 + heavy_n) {
        grp = n - 1;
        r = k - a0;
      } else if (k < a0 + heavy_n + ahead * per) {
        const int k1 = k - a0 - heavy_n;
        const int s = fdiv(k1, o.div_per);
        grp = n - 1 - ahead + s;
        r = k1 - s * per;
      } else {
        grp = n - 1;
        r = k - a0 - heavy_n - ahead * per + heavy_n;   // past the heavy items
      }
      ii = fdiv(r, o.div_group);
      hin = r - ii * group;
    } else if (k < ahead * heavy_n) {   // the first groups' heavy items
      // heavy_n > 0 here (ahead > 0 implies lead > 0)
      grp = fdiv(k, o.div_heavy);
      const int r = k - grp * heavy_n;
      ii = fdiv(r, o.div_group);
      hin = r - ii * group;
    } else {
      // stage j: the heavy items of group j + ahead (if any), then group j's light items
      const int k1 = k - ahead * heavy_n;
      const int full = o.full;
      int j, r;
      bool heavy;
      if (k1 < full) {
        j = fdiv(k1, o.div_per);
        r = k1 - j * per;
        heavy = r < heavy_n;
        if (!heavy) r -= heavy_n;
      } else {
        const int k2 = k1 - full;
        const int s = light_n > 0 ? fdiv(k2, o.div_light) : 0;
        j = (n - ahead) + s;
        r = k2 - s * light_n;
        heavy = false;
      }
      grp = heavy ? j + ahead : j;
      const int rg = fdiv(r, o.div_group);
      ii = (heavy ? 0 : lead) + rg;
      hin = r - rg * group;
    }
    i = o.nb - 1 - ii;
    bh = xcd + 8 * (grp * group + hin);
  } else {
    const int ii = fdiv(L, o.div_bh);
    bh = L - ii * o.BH;
    i = o.nb - 1 - ii;
  }
}

// The same order from its parameters (host checks).
BSATTN_HD void map_item(int L, int BH, int nb, int mode, int group, int lead, int ahead, bool tail,
                        int& bh, int& i) {
  map_item(make_item_order(BH, nb, mode, group, lead, ahead, tail), L, bh, i);
}

}  // namespace bsattn
