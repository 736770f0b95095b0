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

#if defined(__HIPCC__)
#define BSATTN_HD __host__ __device__ __forceinline__
#else
#define BSATTN_HD inline
#endif

namespace bsattn {

BSATTN_HD void map_item(int L, int BH, int nb, int mode, int group, int lead, int ahead, bool tail,
                        int& bh, int& i) {
  if (mode == 1) {
    const int xcd = L & 7;
    const int k = L >> 3;
    const int n = (BH / 8) / group;   // groups on this XCD
    if (lead > nb) lead = nb;
    if (ahead > (tail ? n - 1 : n)) ahead = tail ? n - 1 : n;
    if (lead <= 0 || ahead <= 0) {
      lead = 0;
      ahead = 0;
    }
    const int heavy_n = lead * group;          // look-ahead items per group
    const int light_n = (nb - lead) * group;   // the rest of a group
    const int per = heavy_n + light_n;
    int grp, ii, hin;
    if (tail) {
      // groups 0 .. n-2-ahead | heavy of group n-1 | groups n-1-ahead .. n-2 | light of group n-1
      const int a0 = (n - 1 - ahead) * per;
      int r;
      if (ahead == 0 || k < a0) {
        grp = k / per;
        r = k - grp * per;
      } else if (k < a0 + heavy_n) {
        grp = n - 1;
        r = k - a0;
      } else if (k < a0 + heavy_n + ahead * per) {
        const int k1 = k - a0 - heavy_n;
        const int s = k1 / per;
        grp = n - 1 - ahead + s;
        r = k1 - s * per;
      } else {
        grp = n - 1;
        r = k - a0 - heavy_n - ahead * per + heavy_n;   // past the heavy items
      }
      ii = r / group;
      hin = r - ii * group;
    } else if (k < ahead * heavy_n) {   // the first groups' heavy items
      grp = k / heavy_n;
      const int r = k - grp * heavy_n;
      ii = r / group;
      hin = r - ii * group;
    } else {
      // stage j: the heavy items of group j + ahead (if any), then group j's light items
      const int k1 = k - ahead * heavy_n;
      const int full = (n - ahead) * per;
      int j, r;
      bool heavy;
      if (k1 < full) {
        j = k1 / per;
        r = k1 - j * per;
        heavy = r < heavy_n;
        if (!heavy) r -= heavy_n;
      } else {
        const int k2 = k1 - full;
        const int s = light_n > 0 ? k2 / light_n : 0;
        j = (n - ahead) + s;
        r = k2 - s * light_n;
        heavy = false;
      }
      grp = heavy ? j + ahead : j;
      ii = (heavy ? 0 : lead) + r / group;
      hin = r - (r / group) * group;
    }
    i = nb - 1 - ii;
    bh = xcd + 8 * (grp * group + hin);
  } else {
    const int ii = L / BH;
    bh = L - ii * BH;
    i = nb - 1 - ii;
  }
}

}  // namespace bsattn
