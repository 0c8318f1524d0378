"""Pins of the oracle's dispatch layout and dedup (CPU only).

Against the worked W = 3 example of "Kernel fusion for expert parallelism" (section
"Expert parallelism: dispatch and combine"), the printed distinct-GPU and dedup statistics of
Expert Coupling in MoE Pretraining Table I (contiguous rows, which uniform routing reproduces),
the blog's distinct-rank estimate (section "INC all-to-all phased"), closed forms and invariants.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import moe_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _check_invariants(idx, pi, W, lay):
    N, k = idx.shape
    E = len(pi)
    R = N * k
    assert lay["expert_counts"].sum() == R                       # counts sum to N k
    assert lay["rank_counts"].sum() == R
    assert lay["group_offsets"][-1] == R and lay["rank_offsets"][-1] == R
    # bijection with a correct inverse
    assert sorted(lay["row_of_slot"].tolist()) == list(range(R))
    assert np.array_equal(lay["slot_of_row"][lay["row_of_slot"]], np.arange(R))
    assert np.array_equal(lay["row_of_slot"][lay["slot_of_row"]], np.arange(R))
    # rows sorted by (rank, expert, token) and each group holds exactly its expert's rows
    t = lay["slot_of_row"] // k
    e = idx.reshape(-1)[lay["slot_of_row"]]
    key = [(int(pi[a]), int(a), int(b)) for a, b in zip(e, t)]
    assert key == sorted(key)
    for g, ex in enumerate(lay["group_expert"]):
        lo, hi = lay["group_offsets"][g], lay["group_offsets"][g + 1]
        assert np.all(e[lo:hi] == ex) and hi - lo == lay["expert_counts"][ex]
        assert lay["expert_offsets"][ex] == lo
    for r in range(W):
        lo, hi = lay["rank_offsets"][r], lay["rank_offsets"][r + 1]
        assert np.all(pi[e[lo:hi]] == r)
    # send matrix: row sums = slots of each owner's tokens, column sums = rank counts
    sc = lay["send_counts"]
    assert np.array_equal(sc.sum(1), np.full(W, (N // W) * k))
    assert np.array_equal(sc.sum(0), lay["rank_counts"])
    # dedup: D = sum over tokens of the distinct ranks of its experts (brute force)
    d = [len({int(pi[x]) for x in row}) for row in idx]
    assert lay["D"] == sum(d) == lay["pair_counts"].sum()
    pt, pos = lay["pair_token"], lay["pair_of_slot"]
    for s in range(R):
        tt, j = divmod(s, k)
        p = pos[s]
        assert pt[p] == tt
        assert lay["pair_offsets"][pi[idx[tt, j]]] <= p < lay["pair_offsets"][pi[idx[tt, j]] + 1]
    keys = [(int(np.searchsorted(lay["pair_offsets"], p, "right") - 1), int(pt[p]))
            for p in range(lay["D"])]
    assert keys == sorted(keys) and len(set(keys)) == len(keys)
    assert np.array_equal(lay["pair_send_counts"].sum(0), lay["pair_counts"])
    # every expanded row copies the pair row of its own (token, rank)
    assert np.array_equal(lay["expand_src"], pos[lay["slot_of_row"]])


def test_worked_example():
    g = _load("kf_worked_example.json")
    names = g["tokens"]
    idx = np.array([g["selected_experts"][n] for n in names], np.int32)
    pi = np.array(g["expert_rank"], np.int32)
    W = g["W"]
    lay = O.layout(idx, pi, W)
    _check_invariants(idx, pi, W, lay)
    k = g["k"]
    # per-rank receive sets (the A, C / B, C / A, B groups of the timeline)
    for r in range(W):
        lo, hi = lay["rank_offsets"][r], lay["rank_offsets"][r + 1]
        got = sorted(names[s // k] for s in lay["slot_of_row"][lo:hi])
        assert got == sorted(g["receive_sets"][str(r)])
    # send matrix: a packet per (sender, receiver), the empty ones signal-only
    sc = lay["send_counts"]
    assert sc.size == g["packets_per_collective"]
    zeros = sorted(map(list, np.argwhere(sc == 0).tolist()))
    assert zeros == sorted(g["signal_only_pairs"])
    assert sc.tolist() == [[1, 0, 1], [0, 1, 1], [1, 1, 0]]
    assert lay["row_of_slot"].tolist() == [0, 4, 2, 5, 1, 3]
    # one expert per rank: dedup removes nothing
    assert lay["D"] == 6 and np.array_equal(lay["pair_counts"], lay["rank_counts"])


def test_invariants_random_with_permuted_placement():
    rng = np.random.default_rng(3)
    N, E, k, W = 48, 12, 3, 4
    l = rng.standard_normal((N, E)).astype(np.float32)
    idx, _ = O.route(l, None, k, "softmax")
    pi = O.contiguous_placement(E, W)[rng.permutation(E)]     # a balanced non-contiguous placement
    _check_invariants(idx, pi, W, O.layout(idx, pi, W))


def test_k1_no_duplicates_and_k_equals_e():
    rng = np.random.default_rng(4)
    N, E, W = 32, 8, 4
    l = rng.standard_normal((N, E)).astype(np.float32)
    pi = O.contiguous_placement(E, W)
    lay = O.layout(O.route(l, None, 1, "softmax")[0], pi, W)
    assert lay["D"] == N
    lay = O.layout(O.route(l, None, E, "softmax")[0], pi, W)
    assert lay["D"] == N * W and np.all(lay["expert_counts"] == N)


def test_empty_experts_and_all_tokens_on_one_expert():
    N, E, k, W = 16, 8, 2, 4
    idx = np.tile(np.array([[5, 4]], np.int32), (N, 1))
    pi = O.contiguous_placement(E, W)
    lay = O.layout(idx, pi, W)
    _check_invariants(idx, pi, W, lay)
    assert lay["expert_counts"].tolist() == [0, 0, 0, 0, N, N, 0, 0]
    assert lay["rank_counts"].tolist() == [0, 0, 2 * N, 0]
    assert lay["D"] == N                      # both experts on rank 2: one pair per token


def _uniform_routing(N, E, k, seed):
    rng = np.random.default_rng(seed)
    return O.route(rng.standard_normal((N, E)).astype(np.float32), None, k, "softmax")[0]


def _expected_distinct(E, W, k):
    return W * (1 - math.comb(E - E // W, k) / math.comb(E, k))


@pytest.mark.parametrize("row", _load("ec_table1.json")["rows"][::2])   # contiguous rows
def test_table1_contiguous_rows_under_uniform_routing(row):
    """Uniform routing with contiguous placement reproduces the contiguous rows of Table I."""
    E, k, W = 128, row["topk"], row["EP"]
    N = 16 * 1024
    idx = _uniform_routing(N, E, k, seed=10 + W + k)
    lay = O.layout(idx, O.contiguous_placement(E, W), W)
    gpus = lay["D"] / N
    dedup = 100 * (1 - lay["D"] / (N * k))
    assert abs(gpus - row["gpus"]) < 0.03
    assert abs(dedup - row["dedup"]) < 1.0
    assert abs(gpus - _expected_distinct(E, W, k)) < 0.02
    same = 100 * np.mean([len({int(e) // (E // W) for e in r}) == 1 for r in idx])
    assert abs(same - row["same_gpu"]) < 1.5


def test_distinct_ranks_estimate_single_token():
    g = _load("kf_distinct_ranks.json")
    k, W = g["k"], g["W"]
    E = 64
    approx = W * (1 - (1 - 1 / W) ** (k * g["m_b"]))
    assert round(approx, 1) == g["distinct_ranks"]
    idx = _uniform_routing(20000, E, k, seed=5)
    lay = O.layout(idx, O.contiguous_placement(E, W), W)
    mean_d = lay["D"] / idx.shape[0]
    # distinct experts per token make the exact mean slightly larger than the estimate
    assert abs(mean_d - _expected_distinct(E, W, k)) < 0.02
    assert abs(mean_d - g["distinct_ranks"]) < 0.1


def test_dispatch_rows_dst_rank():
    rng = np.random.default_rng(6)
    N, E, k, W, H = 24, 8, 2, 4, 5
    x = rng.standard_normal((N, H))
    idx = _uniform_routing(N, E, k, 7)
    lay = O.layout(idx, O.contiguous_placement(E, W), W)
    allrows = O.dispatch_rows(x, lay, dedup=False)
    for r in range(W):
        part = O.dispatch_rows(x, lay, dedup=False, dst_rank=r)
        assert np.array_equal(part, allrows[lay["rank_offsets"][r]:lay["rank_offsets"][r + 1]])
    pairs = O.dispatch_rows(x, lay, dedup=True)
    assert pairs.shape[0] == lay["D"]
    assert np.array_equal(pairs[lay["expand_src"]], allrows)
