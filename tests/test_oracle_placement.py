"""Pins of the oracle's correlated placement (Expert Coupling in MoE Pretraining, section V-A
"Correlated Placement" and Appendix A-D Algorithm 1) and of the co-selection counts."""
import itertools

import numpy as np

from oracle import moe_oracle as O


def test_coselect_counts_brute_force():
    idx = np.array([[0, 2], [2, 0], [1, 3], [0, 1]], np.int32)
    Wc = O.coselect_counts(idx, 4)
    want = np.zeros((4, 4), int)
    for row in idx:
        for a, b in itertools.permutations(row.tolist(), 2):
            want[a, b] += 1
    assert np.array_equal(Wc, want) and np.array_equal(Wc, Wc.T) and np.all(np.diag(Wc) == 0)


def _no_positive_swap(Wc, group):
    base = O.intra_weight(Wc, group)
    for a, b in itertools.combinations(range(len(group)), 2):
        if group[a] != group[b]:
            g = group.copy()
            g[a], g[b] = g[b], g[a]
            if O.intra_weight(Wc, g) > base:
                return False
    return True


def test_partition_balanced_local_optimum_random():
    rng = np.random.default_rng(0)
    for E, G in [(8, 2), (12, 3), (16, 4)]:
        Wc = rng.integers(0, 20, size=(E, E))
        Wc = np.triu(Wc, 1)
        Wc = Wc + Wc.T
        group, swaps = O.partition(Wc, G)
        assert np.all(np.bincount(group, minlength=G) == E // G)
        assert _no_positive_swap(Wc, group)
        assert O.intra_weight(Wc, group) >= O.intra_weight(Wc, np.arange(E) // (E // G))


def test_partition_gain_matches_recomputed_weight():
    """Each swap raises the intra-group weight by exactly its gain: replaying the swaps one at a
    time with i_max = 1, 2, ... gives a strictly increasing intra weight."""
    rng = np.random.default_rng(1)
    E, G = 12, 4
    Wc = np.triu(rng.integers(0, 9, size=(E, E)), 1)
    Wc = Wc + Wc.T
    prev = O.intra_weight(Wc, np.arange(E) // (E // G))
    _, total = O.partition(Wc, G)
    for i in range(1, total + 1):
        g, s = O.partition(Wc, G, i_max=i)
        assert s == i
        cur = O.intra_weight(Wc, g)
        assert cur > prev
        prev = cur


def test_partition_small_exhaustive_optimum_reached_from_easy_start():
    # two strong disjoint pairs split across contiguous groups are joined by one swap
    E, G = 4, 2
    Wc = np.zeros((E, E), int)
    Wc[0, 2] = Wc[2, 0] = 10
    Wc[1, 3] = Wc[3, 1] = 10
    group, swaps = O.partition(Wc, G)
    assert swaps == 1 and group[0] == group[2] and group[1] == group[3]
    best = max(O.intra_weight(Wc, np.array(p)) for p in
               set(itertools.permutations([0, 0, 1, 1])))
    assert O.intra_weight(Wc, group) == best


def test_disjoint_hot_pairs_end_on_one_rank():
    rng = np.random.default_rng(2)
    E, G, N = 16, 8, 4000
    perm = rng.permutation(E)
    pairs = perm.reshape(-1, 2)
    idx = pairs[rng.integers(0, len(pairs), N)]
    group, _ = O.partition(O.coselect_counts(idx, E), G)
    assert all(group[a] == group[b] for a, b in pairs)


def test_correlated_placement_raises_dedup():
    """Co-locating co-selected experts lets the dedup dispatcher merge more rows (section V-A)."""
    rng = np.random.default_rng(3)
    E, W, N, k = 16, 8, 3000, 2
    pairs = rng.permutation(E).reshape(-1, 2)
    idx = pairs[rng.integers(0, len(pairs), N)].astype(np.int32)
    contig = O.layout(idx, O.contiguous_placement(E, W), W)
    group, _ = O.partition(O.coselect_counts(idx, E), W)
    corr = O.layout(idx, group, W)
    assert corr["D"] == N < contig["D"]
