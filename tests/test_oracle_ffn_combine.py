"""Pins of the oracle's expert FFN and combine (CPU only).

The MoE output is the gate-weighted sum of the selected experts' outputs plus the shared experts
(FarSkip-Collective section 2.1). "Kernel fusion for expert parallelism" evaluates it as
AllGather-ReduceScatter or as All-to-All; Expert Coupling in MoE Pretraining (section V-A) as a
deduplicated all-to-all with per-(token, rank) weighted partials. All must agree.
"""
import math

import numpy as np

from oracle import moe_oracle as O


def test_swiglu_hand_computed_nonsquare():
    # H = 2, I = 1: gate row [1, 0], up row [0, 1], down column [1, 3]
    x = np.array([[1.0, 2.0]])
    w_gu = np.array([[1.0, 0.0], [0.0, 1.0]])
    w_d = np.array([[1.0], [3.0]])
    s1 = 1.0 / (1.0 + math.exp(-1.0))              # silu(1)
    np.testing.assert_allclose(O.swiglu_expert(x, w_gu, w_d), [[2 * s1, 6 * s1]], rtol=1e-15)
    # gate and up are not interchangeable: silu(2) * 1 differs
    s2 = 2.0 / (1.0 + math.exp(-2.0))
    w_swapped = w_gu[::-1].copy()
    np.testing.assert_allclose(O.swiglu_expert(x, w_swapped, w_d), [[s2, 3 * s2]], rtol=1e-15)


def test_swiglu_shapes_and_zero_up():
    rng = np.random.default_rng(0)
    H, I = 6, 4
    x = rng.standard_normal((5, H))
    w_gu = rng.standard_normal((2 * I, H))
    w_d = rng.standard_normal((H, I))
    assert O.swiglu_expert(x, w_gu, w_d).shape == (5, H)
    w_gu[I:] = 0
    assert np.all(O.swiglu_expert(x, w_gu, w_d) == 0)


def test_swiglu_basis_vectors():
    # x = basis vector e_i picks column i of W_g and W_u; W_d = identity (H = I)
    H = I = 3
    a = np.array([0.0, math.log(3.0), -1.0])
    b = np.array([2.0, 4.0, -5.0])
    w_gu = np.zeros((2 * I, H))
    w_gu[:I, 1] = a
    w_gu[I:, 1] = b
    x = np.array([[0.0, 1.0, 0.0]])
    want = [0.0, math.log(3.0) * 0.75 * 4.0, -1.0 / (1.0 + math.e) * -5.0]
    np.testing.assert_allclose(O.swiglu_expert(x, w_gu, np.eye(3))[0], want, rtol=1e-14,
                               atol=1e-300)


def _small_problem(seed, N=24, H=8, E=6, k=3, W=3, I=5, n_shared=2):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((N, H))
    l = rng.standard_normal((N, E)).astype(np.float32)
    idx, w = O.route(l, None, k, "softmax")
    experts = {e: (rng.standard_normal((2 * I, H)), rng.standard_normal((H, I)))
               for e in range(E)}
    shared = [(rng.standard_normal((2 * I, H)), rng.standard_normal((H, I)))
              for _ in range(n_shared)]
    pi = O.contiguous_placement(E, W)
    return x, idx, w, experts, shared, pi, W


def test_evaluations_agree():
    for pi_perm in (False, True):
        x, idx, w, experts, shared, pi, W = _small_problem(1)
        if pi_perm:
            pi = pi[np.random.default_rng(2).permutation(len(pi))]
        fn = lambda e, rows: O.swiglu_expert(rows, *experts[e])
        shared_fns = [lambda rows, s=s: O.swiglu_expert(rows, *s) for s in shared]
        ref = O.moe_layer(x, idx, w, fn, shared_fns)

        lay = O.layout(idx, pi, W)
        k = idx.shape[1]
        y = O.expert_outputs(x, lay, k, experts)
        sh = np.stack([f(x) for f in shared_fns])
        a2a = O.combine_a2a(y, lay, w, shared=sh)
        agrs, sigma = O.combine_agrs(x, idx, w, pi, W, fn, shared_fns)
        part = O.dedup_partials(y, lay, idx, w, pi)
        dd = O.combine_dedup(part, lay, k, shared=sh)
        scale = np.abs(ref).max()
        for got in (a2a, agrs, dd):
            assert np.abs(got - ref).max() <= 1e-12 * scale
        # AGRS zero partial sums where a rank holds none of the token's experts
        for r in range(W):
            for t in range(x.shape[0]):
                if not any(pi[e] == r for e in idx[t]):
                    assert np.all(sigma[r, t] == 0)
        # the dedup partials are the AGRS partial sums of the pairs
        for p in range(lay["D"]):
            r = int(np.searchsorted(lay["pair_offsets"], p, "right") - 1)
            np.testing.assert_allclose(part[p], sigma[r, lay["pair_token"][p]], rtol=1e-12,
                                       atol=1e-12 * scale)


def test_owner_slice_combine():
    x, idx, w, experts, shared, pi, W = _small_problem(3, n_shared=0)
    lay = O.layout(idx, pi, W)
    y = O.expert_outputs(x, lay, idx.shape[1], experts)
    full = O.combine_a2a(y, lay, w)
    np.testing.assert_array_equal(O.combine_a2a(y, lay, w, 8, 16), full[8:16])


def test_identity_experts_return_x():
    """Renormalised weights sum to 1, so identity experts give out = x."""
    rng = np.random.default_rng(4)
    N, H, E, k, W = 32, 4, 8, 2, 4
    x = rng.standard_normal((N, H))
    idx, w = O.route(rng.standard_normal((N, E)).astype(np.float32), None, k, "softmax")
    lay = O.layout(idx, O.contiguous_placement(E, W), W)
    y = O.expert_outputs(x, lay, k, {}, identity=True)
    np.testing.assert_allclose(O.combine_a2a(y, lay, w), x, rtol=1e-6, atol=1e-6)
    part = O.dedup_partials(y, lay, idx, w, O.contiguous_placement(E, W))
    np.testing.assert_allclose(O.combine_dedup(part, lay, k), x, rtol=1e-6, atol=1e-6)
    # dispatch and combine carry the same rows: one returned row per dispatched row
    assert y.shape[0] == N * k and part.shape[0] == lay["D"]


def test_single_expert_is_dense_mlp():
    """E = k = 1: the layer is one SwiGLU MLP applied to every token (weight 1)."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((10, 6))
    w_gu, w_d = rng.standard_normal((8, 6)), rng.standard_normal((6, 4))
    idx, w = O.route(np.zeros((10, 1), np.float32), None, 1, "softmax")
    out = O.moe_layer(x, idx, w, lambda e, r: O.swiglu_expert(r, w_gu, w_d))
    rowwise = np.stack([O.swiglu_expert(x[i:i + 1], w_gu, w_d)[0] for i in range(10)])
    np.testing.assert_allclose(out, rowwise, rtol=1e-14)
