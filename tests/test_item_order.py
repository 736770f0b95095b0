"""The forward's work-item order (csrc/item_order.hpp), compiled for the host.

map_item must be a bijection from work-group index to (batch*head, query
block); in mode 1 each item must run on the XCD that owns its head
(bh % 8 == L % 8); and the order must be the one the header describes, which
this test builds independently by concatenating lists: per XCD, either the
heavy items (the first `lead` query blocks, descending) of groups 0 ..
ahead-1, then for each group j the heavy items of group j + ahead followed
by group j's remaining query blocks; or (tail) the plain walk with only the
last group's heavy items moved to just before group n - 1 - ahead; heads
interleaved within a group."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
HDR = os.path.join(HERE, "..", "block_sparse_attention_amd", "csrc")

DRIVER = r"""
#include <cstdio>
#include "item_order.hpp"
int main() {
  int BH, nb, mode, group, lead, ahead, tail;
  while (std::scanf("%d %d %d %d %d %d %d", &BH, &nb, &mode, &group, &lead, &ahead, &tail) == 7) {
    for (int L = 0; L < BH * nb; ++L) {
      int bh, i;
      bsattn::map_item(L, BH, nb, mode, group, lead, ahead, tail != 0, bh, i);
      std::printf("%d %d\n", bh, i);
    }
  }
  return 0;
}
"""


DIV_DRIVER = r"""
#include <cstdio>
#include "item_order.hpp"
int main() {
  unsigned d, x;
  while (std::scanf("%u %u", &d, &x) == 2) {
    const bsattn::FastDiv f = bsattn::make_fastdiv(d);
    std::printf("%d\n", bsattn::fdiv((int)x, f));
  }
  return 0;
}
"""


@pytest.fixture(scope="module")
def div_driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    d = tmp_path_factory.mktemp("fdiv")
    src = d / "fdiv.cpp"
    src.write_text(DIV_DRIVER)
    exe = d / "fdiv"
    subprocess.run([gxx, "-O1", "-std=c++17", "-I", HDR, str(src), "-o", str(exe)], check=True)
    return str(exe)


def test_fast_division_is_exact(div_driver):
    """The launch-time divisors' multiply-and-shift quotient equals integer
    division for every dividend in [0, 2^31): checked at the edges (0, 1,
    multiples of d and their neighbours, 2^31 - 1) and on seeded random
    dividends, for every divisor up to 4096 and for large and power-of-two
    divisors."""
    import random
    rng = random.Random(0)
    top = 2 ** 31 - 1
    divisors = list(range(1, 4097)) + [2 ** k for k in range(13, 31)] + [2 ** k + 1 for k in range(13, 31)] \
        + [2 ** k - 1 for k in range(13, 32)] + [rng.randrange(4097, top) for _ in range(300)]
    pairs = []
    for d in divisors:
        xs = {0, 1, d - 1, d, d + 1, top, top - 1, top - (top % d), top - (top % d) - 1}
        q = top // d
        xs |= {q * d, max(0, q * d - 1), (q // 2) * d - 1 if q >= 2 else 0}
        xs |= {rng.randrange(0, top + 1) for _ in range(20)}
        pairs += [(d, x) for x in xs if 0 <= x <= top]
    stdin = "".join(f"{d} {x}\n" for d, x in pairs)
    res = subprocess.run([div_driver], input=stdin, capture_output=True, text=True, check=True)
    got = list(map(int, res.stdout.split()))
    assert len(got) == len(pairs)
    bad = [(d, x, g) for (d, x), g in zip(pairs, got) if g != x // d]
    assert not bad, bad[:5]


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    d = tmp_path_factory.mktemp("order")
    src = d / "order.cpp"
    src.write_text(DRIVER)
    exe = d / "order"
    subprocess.run([gxx, "-O1", "-std=c++17", "-I", HDR, str(src), "-o", str(exe)], check=True)
    return str(exe)


def expected(BH, nb, mode, group, lead, ahead, tail):
    """The order by construction: a list per XCD, then item L = XCD L % 8's (L // 8)-th entry."""
    if mode == 0:
        return [(L % BH, nb - 1 - L // BH) for L in range(BH * nb)]
    per_xcd = BH // 8
    n = per_xcd // group
    lead = min(lead, nb)
    ahead = min(ahead, n - 1 if tail else n)
    if lead <= 0 or ahead <= 0:
        lead = ahead = 0
    out = [None] * (BH * nb)
    for xcd in range(8):
        def items(grp, ii_range):
            return [(xcd + 8 * (grp * group + h), nb - 1 - ii) for ii in ii_range for h in range(group)]
        seq = []
        if tail:
            for j in range(n - 1):
                if j == n - 1 - ahead:
                    seq += items(n - 1, range(lead))
                seq += items(j, range(nb))
            seq += items(n - 1, range(lead, nb) if ahead else range(nb))
        else:
            for grp in range(ahead):
                seq += items(grp, range(lead))
            for j in range(n):
                if j + ahead < n and ahead > 0:
                    seq += items(j + ahead, range(lead))
                seq += items(j, range(lead, nb))
        assert len(seq) == per_xcd * nb
        for k, it in enumerate(seq):
            out[8 * k + xcd] = it
    return out


CASES = []
for BH in (8, 16, 64, 128, 256):
    for nb in (1, 2, 3, 7, 64, 129):
        per_xcd = BH // 8
        for group in [g for g in range(1, per_xcd + 1) if per_xcd % g == 0][:4]:
            for lead, ahead in ((0, 0), (2, 0), (0, 2), (1, 1), (2, 2), (2, 3), (4, 1), (300, 2), (2, 100)):
                for tail in (0, 1):
                    CASES.append((BH, nb, 1, group, lead, ahead, tail))
    for nb in (1, 5, 64):
        CASES.append((BH, nb, 0, 1, 0, 0, 0))
CASES.append((24, 33, 0, 1, 0, 0, 0))   # batch*heads not a multiple of 8: mode 0
CASES.append((32, 256, 1, 1, 2, 4, 1))  # B1 H32 S16384: the long-row workload's order
CASES.append((32, 128, 1, 1, 0, 0, 0))  # its long rows' helpers (query blocks 128 .. 255)


def test_order_is_the_constructed_one_and_a_bijection(driver):
    stdin = "".join(" ".join(map(str, c)) + "\n" for c in CASES)
    res = subprocess.run([driver], input=stdin, capture_output=True, text=True, check=True)
    rows = [tuple(map(int, l.split())) for l in res.stdout.splitlines()]
    pos = 0
    for BH, nb, mode, group, lead, ahead, tail in CASES:
        got = rows[pos:pos + BH * nb]
        pos += BH * nb
        want = expected(BH, nb, mode, group, lead, ahead, tail)
        assert got == want, (BH, nb, mode, group, lead, ahead, tail)
        assert len(set(got)) == BH * nb   # every item exactly once
        if mode == 1:
            assert all(bh % 8 == L % 8 for L, (bh, _) in enumerate(got))
    assert pos == len(rows)


def test_heavy_rows_come_early(driver):
    """B4 H32 with 128 query blocks, one head per group: without the look-ahead
    the last head's two heaviest rows follow every row of the head before it;
    with a look-ahead of two groups they precede the light rows of the head
    three from the end."""
    BH, nb, group = 128, 128, 1
    n = BH // 8 // group

    def xcd0(lead, ahead, tail=0):
        stdin = f"{BH} {nb} 1 {group} {lead} {ahead} {tail}\n"
        res = subprocess.run([driver], input=stdin, capture_output=True, text=True, check=True)
        seq = [tuple(map(int, l.split())) for l in res.stdout.splitlines()]
        return [seq[8 * k] for k in range(BH * nb // 8)]

    def pos(seq, head, rows):
        return [k for k, (bh, i) in enumerate(seq) if bh == 8 * head and i in rows]

    heavy, light = set(range(nb - 2, nb)), set(range(nb - 2))
    plain = xcd0(0, 0)
    assert min(pos(plain, n - 1, heavy)) > max(pos(plain, n - 2, light))
    early = xcd0(2, 2)
    assert max(pos(early, n - 1, heavy)) < min(pos(early, n - 3, light))
    # tail only: the last head's heavy rows just before head n - 5; every other head in plain order
    tail = xcd0(2, 4, 1)
    assert max(pos(tail, n - 6, light)) < min(pos(tail, n - 1, heavy))
    assert max(pos(tail, n - 1, heavy)) < min(pos(tail, n - 5, light | heavy))
    for h in range(n - 1):
        assert pos(tail, h, heavy | light) == pos(plain, h, heavy | light) or h >= n - 5
