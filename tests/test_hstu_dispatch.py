"""Index math of the XCD-balanced dispatch of the jagged HSTU kernel (CPU).

The d = 64 HSTU kernel maps its workgroups to (sequence, head, query block)
items as follows (when B <= 64 and 8 <= B*H <= 512):

* sequences are ranked by length, longest first, ties by index;
* the (sequence, head) pairs in rank order (rank-major, head-minor) are dealt
  to the 8 XCDs in snake order: sorted pair i goes to XCD c if i = 8r + c with
  r even, to XCD 7 - c if r is odd; pair k of XCD x is sorted pair
  8k + (k even ? x : 7 - x);
* workgroup w runs on XCD w % 8 and takes entry w // 8 of that XCD's list of
  existing blocks (block q of a pair exists if 64 q < L), heaviest first:
  block index descending, then pair k ascending; workgroups past the list have
  no item.  The grid is 8 * ceil(B*H / 8) * nqb.

The kernel finds its entry without building the list: lane k holds pair k's
block count nb_k (non-increasing in k, the pairs being in length order); blocks
nb_{k+1} .. nb_k - 1 exist for pairs 0 .. k, which makes (nb_k - nb_{k+1})(k+1)
entries; a prefix sum over the lanes locates w // 8.  `lane_parallel` below
restates that arithmetic and `reference_lists` builds the lists directly;
they must agree.

Checked here by enumeration: every existing item is taken by exactly one
workgroup, every pair's blocks stay on one XCD, each XCD's list is in
heaviest-first order with no empty entries before its end, and the quadratic
work per XCD is balanced on the jagged workload.  The kernel itself is checked
against the oracle by the GPU tests.
"""

import numpy as np
import pytest


def _order(lengths, N):
    L = [min(v, N) for v in lengths]
    return L, sorted(range(len(L)), key=lambda b: (-L[b], b))  # rank -> sequence


def _pair_of(x, k):
    return 8 * k + ((7 - x) if k % 2 else x)


def reference_lists(lengths, H, N):
    """Per XCD, the list of its existing (sequence, head, block) items, built directly."""
    L, order = _order(lengths, N)
    npairs = len(L) * H
    lists = []
    for x in range(8):
        pairs = []
        k = 0
        while _pair_of(x, k) < npairs:
            srank, h = divmod(_pair_of(x, k), H)
            pairs.append((order[srank], h))
            k += 1
        nqb = max(1, (N + 63) // 64)
        lst = []
        for q in reversed(range(nqb)):
            for b, h in pairs:
                if 64 * q < L[b]:
                    lst.append((b, h, q))
        lists.append(lst)
    return lists


def lane_parallel(lengths, H, N, w):
    """The kernel's arithmetic for workgroup w: its item, or None."""
    L, order = _order(lengths, N)
    B = len(L)
    npairs = B * H
    len_by_rank = np.full(64, -1)
    len_by_rank[:B] = [L[order[r]] for r in range(B)]
    lanes = np.arange(64)
    x, u = w & 7, w >> 3
    ik = 8 * lanes + np.where(lanes & 1, 7 - x, x)
    nb = np.where(ik < npairs, (len_by_rank[np.minimum(ik // H, 63)] + 63) >> 6, 0)
    nbn = np.where(lanes < 63, nb[(lanes + 1) & 63], 0)
    cnt = (nb - nbn) * (lanes + 1)
    pre = np.cumsum(cnt)
    hit = np.nonzero(pre > u)[0]
    if len(hit) == 0:
        return None
    k = int(hit[0])
    v = u - int(pre[k] - cnt[k])
    q, j = divmod(v, k + 1)
    srank, h = divmod(_pair_of(x, j), H)
    return (order[srank], h, int(nb[k]) - 1 - q)


def dispatch(lengths, H, N):
    nqb = max(1, (N + 63) // 64)
    npairs = len(lengths) * H
    grid = 8 * ((npairs + 7) // 8) * nqb
    items = {}
    per_xcd = [[] for _ in range(8)]
    for w in range(grid):
        it = lane_parallel(lengths, H, N, w)
        if it is None:
            continue
        assert it not in items, it
        items[it] = w % 8
        per_xcd[w % 8].append((w // 8, it))
    return items, per_xcd


CASES = [(1, 8), (2, 4), (3, 3), (6, 3), (16, 4), (5, 7), (64, 1), (64, 2), (13, 5), (7, 16), (64, 8)]


@pytest.mark.parametrize("B,H", CASES)
def test_every_item_exactly_once(B, H):
    rng = np.random.default_rng(B * 100 + H)
    for trial in range(4):
        lengths = [int(v) for v in rng.integers(0, 400, B)]
        if trial == 0:
            lengths = [0] * (B - 1) + [70]  # empty sequences
        if trial == 1:
            lengths = [200] * B  # equal lengths
        N = max(lengths)
        items, per_xcd = dispatch(lengths, H, N)
        want = {(b, h, q) for b in range(B) for h in range(H) for q in range((lengths[b] + 63) // 64)}
        assert set(items) == want
        # all blocks of one (sequence, head) pair on one XCD
        for b in range(B):
            for h in range(H):
                assert len({items[(b, h, q)] for q in range((lengths[b] + 63) // 64)}) <= 1
        # the kernel's arithmetic gives the directly built lists, with entries
        # 0 .. len-1 of each XCD taken and nothing after
        ref = reference_lists(lengths, H, N)
        for x in range(8):
            assert [u for u, _ in per_xcd[x]] == list(range(len(ref[x])))
            assert [it for _, it in per_xcd[x]] == ref[x]
            qs = [q for _, (_, _, q) in per_xcd[x]]
            assert qs == sorted(qs, reverse=True)  # heaviest (last) blocks first


def test_sequences_past_the_length_bound_are_clamped():
    # lengths above N (the launch's maximum) count N rows, as the kernel's clamp does
    items, _ = dispatch([500, 90, 30], 4, 128)
    assert {q for (b, h, q) in items if b == 0} == {0, 1}


def test_ties_are_ranked_by_index():
    items, _ = dispatch([100, 100, 100, 100, 100, 100, 100, 100], 1, 128)
    # equal lengths: sequence b is rank b, dealt to XCD b
    for b in range(8):
        assert items[(b, 0, 0)] == b


def test_jagged_workload_is_balanced_over_xcds():
    from synthgen import workloads as W

    c = W.HSTU_JAGGED
    x = W.jagged_inputs(c)
    lengths = [int(v) for v in x.lengths]
    N = max(lengths)
    items, per_xcd = dispatch(lengths, c.H, N)
    load = np.zeros(8)
    for (b, h, q), xcd in items.items():
        load[xcd] += (min(lengths[b], (q + 1) * 64) + 31) // 32  # key tiles of the block
    assert load.max() / load.mean() < 1.05, load / load.mean()
    # the XCDs' lists are near-equal in length too, so the in-order start of the
    # workgroups hands every XCD a block at the same pace
    n = np.array([len(p) for p in per_xcd])
    assert n.max() - n.min() <= 0.05 * n.mean()
    # the mapping it replaces (pairs b*H + h in blocks of eight per XCD) is far worse
    nqb = (N + 63) // 64
    naive = np.zeros(8)
    for b in range(len(lengths)):
        for h in range(c.H):
            for q in range(nqb):
                L = lengths[b]
                if q * 64 < L:
                    naive[(b * c.H + h) // 8] += (min(L, (q + 1) * 64) + 31) // 32
    assert naive.max() / naive.mean() > 1.3
