"""Index math of the decode work partition (CPU).

The split and combine kernels of ``attn_decode`` share one partition of the
work, computed independently in each kernel from ``seqlens_k``:

* per kv head, the 32-key blocks of all sequences are laid end to end;
  sequence b holds blocks [P_b, P_b + nb_b), nb_b = ceil(L_b / 32),
  T = sum of nb_b;
* with W = B * splits items and W' = min(W, T), item w takes blocks
  [floor(w T / W'), floor((w + 1) T / W'));
* the split kernel writes the partial of (sequence b, item w) to slot w + b;
* the combine kernel reads, for sequence b, the slots of items
  wf = floor(((P_b + 1) W' - 1) / T) .. wl = floor(((P_b + nb_b) W' - 1) / T).

The kernels rely on three facts, checked here by enumeration over random
length sets (empty sequences, T < W, more than 64 sequences, long and short
mixes): every block is covered by exactly one item; the slots written are
distinct and below B * (splits + 1); and the items that touch sequence b are
exactly wf .. wl, so the combine reads every partial of b and nothing else.
The GPU tests check the kernels themselves against the oracle on such shapes.
"""

import numpy as np
import pytest


def partition(lengths, splits):
    nb = [(int(L) + 31) // 32 for L in lengths]
    B = len(nb)
    T = sum(nb)
    P = np.concatenate([[0], np.cumsum(nb)]).astype(int)
    W = B * splits
    Wp = min(W, T)
    writes = []  # (item, sequence, first block, end block) of each segment
    for w in range(Wp):
        lo, hi = w * T // Wp, (w + 1) * T // Wp
        for b in range(B):
            s0, s1 = max(P[b], lo), min(P[b] + nb[b], hi)
            if s0 < s1:
                writes.append((w, b, s0, s1))
    return nb, P, T, Wp, writes


def check(lengths, splits):
    nb, P, T, Wp, writes = partition(lengths, splits)
    B = len(lengths)
    # every block covered exactly once
    cover = np.zeros(T, dtype=int)
    for _, _, s0, s1 in writes:
        cover[s0:s1] += 1
    assert np.all(cover == 1)
    # slots distinct and in range
    slots = [w + b for w, b, _, _ in writes]
    assert len(set(slots)) == len(slots)
    assert all(0 <= s < B * (splits + 1) for s in slots)
    # the combine's range equals the items touching each sequence
    for b in range(B):
        touching = sorted(w for w, bb, _, _ in writes if bb == b)
        if nb[b] == 0:
            assert touching == []
            continue
        wf = ((P[b] + 1) * Wp - 1) // T
        wl = ((P[b] + nb[b]) * Wp - 1) // T
        assert touching == list(range(wf, wl + 1)), (b, touching, wf, wl)


@pytest.mark.parametrize("seed", range(60))
def test_partition_random_lengths(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 140))
    kind = seed % 4
    if kind == 0:    # the decode workload's mix
        lengths = rng.integers(16384, 32769, B)
    elif kind == 1:  # short sequences and empty ones: often T < W
        lengths = rng.integers(0, 100, B)
    elif kind == 2:  # one long sequence among short ones
        lengths = rng.integers(0, 64, B)
        lengths[rng.integers(0, B)] = int(rng.integers(10000, 200000))
    else:            # anything
        lengths = rng.integers(0, 5000, B) * (rng.random(B) < 0.8)
    for splits in (1, 2, 3, 6, 16, 64):
        check(lengths, splits)


def test_partition_edge_cases():
    check([0], 1)
    check([0, 0, 0], 64)
    check([1], 64)                 # T = 1 < W
    check([32, 33, 31], 2)
    check([5] * 70, 1)             # more sequences than a wave's 64 lanes
    check([0] * 65 + [4096], 16)
    check([32768] * 16, 6)         # equal lengths: exactly `splits` items each
    _, _, _, _, w = partition([32768] * 16, 6)
    per_seq = [sum(1 for _, b, _, _ in w if b == s) for s in range(16)]
    assert per_seq == [6] * 16
