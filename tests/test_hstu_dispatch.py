"""Index math of the XCD-balanced dispatch of the jagged HSTU kernel (CPU).

The d = 64 HSTU kernel maps its workgroups to (sequence, head, query block)
items as follows (when B <= 64 and B*H >= 8):

* sequences are ranked by length, longest first, ties by index;
* the (sequence, head) pairs in rank order (rank-major, head-minor) are dealt
  to the 8 XCDs in snake order: sorted pair i goes to XCD c if i = 8r + c with
  r even, to XCD 7 - c if r is odd;
* workgroup w runs on XCD w % 8 at rank u = w // 8 there; with n_x pairs on
  XCD x it takes pair u % n_x (in dealing order) and query block
  nqb - 1 - u // n_x; the grid is 8 * ceil(B*H / 8) * nqb.

Checked here by enumeration: every (sequence, head, block) item is taken by
exactly one workgroup, every workgroup's item lies on its own XCD, and the
quadratic work per XCD is balanced on the jagged workload.  The kernel itself
is checked against the oracle by the GPU tests.
"""

import numpy as np
import pytest


def dispatch(lengths, H, nqb):
    B = len(lengths)
    order = sorted(range(B), key=lambda b: (-lengths[b], b))  # rank -> sequence
    npairs = B * H
    full, rem = divmod(npairs, 8)
    grid = 8 * ((npairs + 7) // 8) * nqb
    items = {}
    for w in range(grid):
        x, u = w % 8, w // 8
        n_x = full + (1 if ((7 - x) if full % 2 else x) < rem else 0)
        if n_x == 0:
            continue
        blk, j = divmod(u, n_x)
        if blk >= nqb:
            continue
        i = 8 * j + ((7 - x) if j % 2 else x)
        assert i < npairs
        srank, h = divmod(i, H)
        b = order[srank]
        qb = nqb - 1 - blk
        key = (b, h, qb)
        assert key not in items, key
        items[key] = x
    return items


@pytest.mark.parametrize("B,H", [(1, 8), (2, 4), (3, 3), (6, 3), (16, 4), (5, 7), (64, 1), (64, 2), (13, 5)])
def test_every_item_exactly_once(B, H):
    rng = np.random.default_rng(B * 100 + H)
    lengths = [int(v) for v in rng.integers(0, 400, B)]
    nqb = max(1, (max(lengths) + 63) // 64)
    items = dispatch(lengths, H, nqb)
    assert set(items) == {(b, h, q) for b in range(B) for h in range(H) for q in range(nqb)}
    # all blocks of one (sequence, head) pair on one XCD
    for b in range(B):
        for h in range(H):
            assert len({items[(b, h, q)] for q in range(nqb)}) == 1


def test_ties_are_ranked_by_index():
    items = dispatch([100, 100, 100, 100, 100, 100, 100, 100], 1, 2)
    # equal lengths: sequence b is rank b, dealt to XCD b
    for b in range(8):
        assert items[(b, 0, 0)] == b


def test_jagged_workload_is_balanced_over_xcds():
    from synthgen import workloads as W

    c = W.HSTU_JAGGED
    x = W.jagged_inputs(c)
    lengths = [int(v) for v in x.lengths]
    nqb = (max(lengths) + 63) // 64
    items = dispatch(lengths, c.H, nqb)
    load = np.zeros(8)
    for (b, h, q), xcd in items.items():
        L = lengths[b]
        if q * 64 < L:
            load[xcd] += (min(L, (q + 1) * 64) + 31) // 32  # key tiles of the block
    assert load.max() / load.mean() < 1.05, load / load.mean()
    # the mapping it replaces (pairs b*H + h in blocks of eight per XCD) is far worse
    naive = np.zeros(8)
    for b in range(len(lengths)):
        for h in range(c.H):
            for q in range(nqb):
                L = lengths[b]
                if q * 64 < L:
                    naive[(b * c.H + h) // 8] += (min(L, (q + 1) * 64) + 31) // 32
    assert naive.max() / naive.mean() > 1.3
