"""Pins of the token-shuffle planner oracle (Expert Coupling in MoE Pretraining, section V-B and
Algorithm 2) against brute force, closed forms, a hand example and properties of the greedy."""

import numpy as np
import pytest

from dispatch_expert_gemm_amd import workloads as WL
from oracle import moe_oracle as O


def _random_trace(rng, T, E, k):
    sets = [np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]) for _ in range(3)]
    return [s.astype(np.int32) for s in sets]


def test_fit_matches_brute_force_counts():
    rng = np.random.default_rng(3)
    T, E, k, P = 60, 6, 2, 3
    p2, p1, cur = _random_trace(rng, T, E, k)
    placement = rng.permutation(np.arange(E) % P).astype(np.int32)
    F, S, n = O.shuffle_fit(p2, p1, cur, placement, P)
    fc = np.zeros((E, P), np.int64)
    sc = np.zeros((E, E, P), np.int64)
    nc = np.zeros((E, E), np.int64)
    for t in range(T):
        for e in p1[t]:
            for x in cur[t]:
                fc[e, placement[x]] += 1
            for e2 in p2[t]:
                nc[e2, e] += 1
                for x in cur[t]:
                    sc[e2, e, placement[x]] += 1
    assert np.array_equal(n, nc)
    for e in range(E):
        tot = fc[e].sum()
        want = (fc[e].astype(np.float32) / np.float32(tot)) if tot else np.full(P, 1 / P, np.float32)
        assert np.array_equal(F[e], want.astype(np.float32))
        for e2 in range(E):
            tot = sc[e2, e].sum()
            want = sc[e2, e].astype(np.float32) / np.float32(tot) if tot else np.zeros(P, np.float32)
            assert np.array_equal(S[e2, e], want)
    assert n.sum() == T * k * k
    assert np.allclose(F.sum(1), 1.0, atol=1e-6)


def test_unused_expert_rows():
    # expert 3 never used at m-1: uniform row; pairs never seen: zero rows and zero support
    p2 = np.array([[0], [1]], np.int32)
    p1 = np.array([[1], [2]], np.int32)
    cur = np.array([[0], [3]], np.int32)
    F, S, n = O.shuffle_fit(p2, p1, cur, np.array([0, 0, 1, 1], np.int32), 2)
    assert np.array_equal(F[3], np.float32([0.5, 0.5]))
    assert np.array_equal(F[1], np.float32([1, 0])) and np.array_equal(F[2], np.float32([0, 1]))
    assert n[0, 1] == 1 and n[1, 2] == 1 and n.sum() == 2
    assert np.array_equal(S[0, 2], np.float32([0, 0]))
    assert np.array_equal(S[1, 2], np.float32([0, 1]))


def test_predict_back_off_weight_by_hand():
    # one token, k = 1: d = (1 - w) F[e] + w S[e', e], w = min(n / (n + beta), w_max)
    F = np.array([[0.5, 0.5], [0.2, 0.8]], np.float32)
    S = np.zeros((2, 2, 2), np.float32)
    S[0, 1] = [0.9, 0.1]
    n = np.array([[0, 3], [0, 0]], np.int32)
    p2, p1 = np.array([[0]]), np.array([[1]])
    d, conf = O.shuffle_predict(p2, p1, F, S, n, beta=1.0, w_max=1.0)     # w = 3/4
    want = 0.25 * np.array([0.2, 0.8]) + 0.75 * np.array([0.9, 0.1])
    assert np.allclose(d[0], want / want.sum(), rtol=1e-7)
    assert np.isclose(conf[0], abs(want[0] - want[1]) / want.sum())
    d, _ = O.shuffle_predict(p2, p1, F, S, n, beta=1.0, w_max=0.5)        # capped at 1/2
    want = 0.5 * np.array([0.2, 0.8]) + 0.5 * np.array([0.9, 0.1])
    assert np.allclose(d[0], want, rtol=1e-7)
    n0 = np.zeros_like(n)                                                  # no support: F only
    d, _ = O.shuffle_predict(p2, p1, F, S, n0, beta=0.0, w_max=1.0)
    assert np.allclose(d[0], [0.2, 0.8], rtol=1e-7)


def test_predict_limits():
    c = WL.ShuffleTrace("t", 5, 512, 16, 3, 4, 8, 4, 0.7, 2048)
    fp2, fp1, fcur = WL.gen_shuffle_trace(c, "fit")
    placement = (np.arange(16) // 4).astype(np.int32)
    F, S, n = O.shuffle_fit(fp2, fp1, fcur, placement, 4)
    p2, p1, _ = WL.gen_shuffle_trace(c, "eval")
    # w_max = 0: first order only, d_t = mean of F over the token's m-1 experts
    d, _ = O.shuffle_predict(p2, p1, F, S, n, beta=4.0, w_max=0.0)
    want = F.astype(np.float64)[p1].mean(1)
    assert np.allclose(d, want / want.sum(1, keepdims=True), rtol=1e-12)
    # beta = 0, w_max = 1: a pair seen in the trace uses its second-order row alone
    d, _ = O.shuffle_predict(fp2, fp1, F, S, n, beta=0.0, w_max=1.0)
    want = S.astype(np.float64)[fp2[:, :, None], fp1[:, None, :]].reshape(len(fp1), -1, 4).mean(1)
    assert np.allclose(d, want / want.sum(1, keepdims=True), rtol=1e-12)
    assert np.allclose(d.sum(1), 1.0)


def test_assign_hand_example():
    d = np.array([[0.9, 0.1], [0.6, 0.4], [0.8, 0.2], [0.7, 0.3]])
    conf = np.array([0.8, 0.2, 0.6, 0.4])
    # order t0, t2, t3, t1; rank 0 fills with t0 and t2, so t3 and t1 go to rank 1
    assert O.shuffle_assign(d, conf, 2).tolist() == [0, 1, 0, 1]
    # equal confidence: lower token first; equal d: lower rank first
    d = np.array([[0.5, 0.5], [0.5, 0.5], [0.5, 0.5], [0.5, 0.5]])
    assert O.shuffle_assign(d, np.zeros(4), 2).tolist() == [0, 0, 1, 1]


def test_assign_properties_random():
    rng = np.random.default_rng(11)
    T, P = 240, 6
    d = rng.dirichlet(np.full(P, 0.5), size=T)
    top = np.sort(d, 1)
    conf = top[:, -1] - top[:, -2]
    owner = O.shuffle_assign(d, conf, P)
    assert np.bincount(owner, minlength=P).tolist() == [T // P] * P
    order = np.lexsort((np.arange(T), -conf))
    pos = np.empty(T, np.int64)
    pos[order] = np.arange(T)
    best = d.argmax(1)
    for t in range(T):
        if owner[t] != best[t]:
            # its best rank was filled by more confident tokens
            holders = np.nonzero(owner == best[t])[0]
            assert len(holders) == T // P and (pos[holders] < pos[t]).all()
            # and it took the best rank among those still open at its turn
            open_ranks = [r for r in range(P)
                          if (pos[np.nonzero(owner == r)[0]] < pos[t]).sum() < T // P]
            assert owner[t] == max(open_ranks, key=lambda r: (d[t, r], -r))
    # when every rank is the best rank of exactly T/P tokens the cap never binds
    d = np.full((T, P), 0.1)
    d[np.arange(T), np.arange(T) % P] = 0.5
    assert np.array_equal(O.shuffle_assign(d, rng.random(T), P), np.arange(T) % P)


def test_assign_brute_force_tiny():
    # all assignment orders of a tiny case: the greedy result equals the sequential definition
    rng = np.random.default_rng(2)
    T, P = 6, 3
    for _ in range(20):
        d = rng.random((T, P))
        conf = rng.integers(0, 3, T).astype(float)      # many equal confidences
        cap = [T // P] * P
        want = [None] * T
        for t in sorted(range(T), key=lambda t: (-conf[t], t)):
            r = max((r for r in range(P) if cap[r] > 0), key=lambda r: (d[t, r], -r))
            want[t] = r
            cap[r] -= 1
        assert O.shuffle_assign(d, conf, P).tolist() == want


def test_order_and_inverse():
    owner = np.array([2, 0, 1, 0, 2, 1], np.int32)
    order, inverse = O.shuffle_order(owner, 3)
    assert order.tolist() == [1, 3, 2, 5, 0, 4]
    assert np.array_equal(order[inverse], np.arange(6))
    assert np.array_equal(owner[order], [0, 0, 1, 1, 2, 2])


def test_planted_routing_reaches_full_locality():
    # every token's position-m experts sit on one rank that its m-1 experts determine, and the
    # ranks are equally popular: the planner places every token with all its experts
    E, P, k, T = 8, 4, 2, 64
    rng = np.random.default_rng(5)
    cls = rng.permutation(np.arange(T) % P)
    sets = np.stack([2 * cls, 2 * cls + 1], 1).astype(np.int32)   # class c: experts 2c, 2c+1
    placement = (np.arange(E) // 2).astype(np.int32)
    F, S, n = O.shuffle_fit(sets, sets, sets, placement, P)
    d, conf = O.shuffle_predict(sets, sets, F, S, n, beta=1.0, w_max=0.9)
    owner = O.shuffle_assign(d, conf, P)
    assert np.array_equal(owner, cls)
    assert O.shuffle_locality(sets, placement, owner) == 1.0
    # the canonical contiguous slices find about 1 / P of the slots local
    canon = np.arange(T) // (T // P)
    assert O.shuffle_locality(sets, placement, canon) < 0.5


@pytest.mark.parametrize("name", ["ec-top2-p8", "ec-top6-p16"])
def test_planner_raises_locality_on_correlated_traces(name):
    # stand-in traces under correlated placement (Algorithm 1 on the trace's position-m
    # co-selection): tables fit on one trace raise the locality of another well above the
    # canonical 1/P of contiguous sequence slices ([EC] section VI-C: 12.5% at EP8 without it)
    c = WL.SHUFFLE_TRACES[name]
    c = WL.ShuffleTrace(c.name, c.seed, 2048, c.E, c.k, c.P, c.classes, c.pref, c.rho, 16384)
    fit = WL.gen_shuffle_trace(c, "fit")
    placement, _ = O.partition(O.coselect_counts(fit[2], c.E), c.P)
    F, S, n = O.shuffle_fit(*fit, placement, c.P)
    p2, p1, cur = WL.gen_shuffle_trace(c, "eval")
    d, conf = O.shuffle_predict(p2, p1, F, S, n, beta=8.0, w_max=0.9)
    owner = O.shuffle_assign(d, conf, c.P)
    canon = np.arange(c.T) // (c.T // c.P)
    base = O.shuffle_locality(cur, placement, canon)
    got = O.shuffle_locality(cur, placement, owner)
    assert abs(base - 1 / c.P) < 0.02
    assert got > base + 0.2
