"""Pins for the split-count heuristic oracle: hand-worked values (CPU only)."""
import os

from oracle import heuristic as oh

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_worked_values():
    n = 0
    for line in open(os.path.join(GOLD, "num_splits_worked.txt")):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        tm, sms, nn, nm, size, causal, mx, want = (int(x) for x in line.split())
        assert oh.num_splits_heuristic(tm, sms, nn, nm, size, bool(causal), mx) == want, line
        n += 1
    assert n == 10


def test_decode_wrapper_on_the_decode_workload():
    # batch 8, 32 query heads over 8 KV heads, D 128, 64 selected blocks, 256 CUs:
    # one m-block per (batch, KV head) -> 64 m-blocks -> eff .25 .5 .75 1 -> 4
    assert oh.decode_num_splits(8, 32, 8, 64, 128, 256) == 4
    # the guide's regression size, batch 1: 8 m-blocks on 256 CUs, eff(s) = s/32 for s <= 32
    # (1.0 at s = 32), so the first s with eff >= .85 is 28
    assert oh.decode_num_splits(1, 32, 8, 64, 128, 256) == 28
