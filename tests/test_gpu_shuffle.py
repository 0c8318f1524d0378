"""GPU parity of the token-shuffle planner (Expert Coupling in MoE Pretraining, section V-B and
Algorithm 2) against the CPU oracle: tables bit-exact, predicted distributions and confidences
at fp32 tolerance, and owners, order and inverse bit-exact against the oracle's greedy run on
the GPU's own distributions and confidences (the assignment is decided in the kernel's fp32)."""
import numpy as np
import pytest
import torch

from dispatch_expert_gemm_amd import moe
from dispatch_expert_gemm_amd import workloads as WL
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu
DEV = "cuda"
D_RTOL = 2e-6          # fp32 sums of at most k^2 = 256 terms, normalised


def _trace(name, T, fit_tokens, **kw):
    c = WL.SHUFFLE_TRACES[name]
    c = WL.ShuffleTrace(c.name, c.seed, T, kw.get("E", c.E), kw.get("k", c.k), kw.get("P", c.P),
                        c.classes, c.pref, c.rho, fit_tokens)
    return c, WL.gen_shuffle_trace(c, "fit"), WL.gen_shuffle_trace(c, "eval")


def _d(*arrs):
    return [torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in arrs]


def _check_plan(p2, p1, F, S, n, beta, w_max, P):
    d, conf, owner, order, inverse = moe.moe_shuffle_plan(*_d(p2, p1, F, S, n), beta, w_max)
    torch.cuda.synchronize()
    d, conf = d.cpu().numpy(), conf.cpu().numpy()
    owner, order, inverse = owner.cpu().numpy(), order.cpu().numpy(), inverse.cpu().numpy()
    d_ref, conf_ref = O.shuffle_predict(p2, p1, F, S, n, beta, w_max)
    assert np.abs(d - d_ref).max() <= D_RTOL * max(1.0, np.abs(d_ref).max())
    assert np.abs(conf - conf_ref).max() <= 4 * D_RTOL
    want = O.shuffle_assign(d.astype(np.float64), conf.astype(np.float64), P)
    assert np.array_equal(owner, want)
    o_ref, i_ref = O.shuffle_order(want, P)
    assert np.array_equal(order, o_ref) and np.array_equal(inverse, i_ref)
    assert np.bincount(owner, minlength=P).tolist() == [len(owner) // P] * P
    return owner


@pytest.mark.parametrize("name,P", [("ec-top2-p8", 8), ("ec-top6-p8", 8), ("ec-top6-p16", 16),
                                    ("ec-top2-p8", 64)])
def test_fit_bit_exact(name, P):
    c, fit, _ = _trace(name, 512, 8192, P=P)
    rng = np.random.default_rng(P)
    placement = rng.permutation(np.arange(c.E) % P).astype(np.int32)
    F, S, n = moe.moe_shuffle_fit(*_d(*fit, placement), c.E, P)
    F_ref, S_ref, n_ref = O.shuffle_fit(*fit, placement, P)
    assert np.array_equal(n.cpu().numpy(), n_ref)
    assert np.array_equal(F.cpu().numpy(), F_ref)
    assert np.array_equal(S.cpu().numpy(), S_ref)


@pytest.mark.parametrize("name,T,beta,w_max", [("ec-top2-p8", 4096, 8.0, 0.9),
                                               ("ec-top6-p8", 2048, 8.0, 0.9),
                                               ("ec-top6-p16", 2048, 2.0, 0.5),
                                               ("ec-top2-p8", 1000, 0.0, 1.0),
                                               ("ec-top6-p8", 968, 4.0, 0.0)])
def test_plan_matches_oracle(name, T, beta, w_max):
    c, fit, (p2, p1, cur) = _trace(name, T, 8192)
    grp, _ = O.partition(O.coselect_counts(fit[2], c.E), c.P)
    F, S, n = O.shuffle_fit(*fit, grp, c.P)
    owner = _check_plan(p2, p1, F, S, n, beta, w_max, c.P)
    canon = np.arange(T) // (T // c.P)
    if w_max > 0:
        assert O.shuffle_locality(cur, grp, owner) > O.shuffle_locality(cur, grp, canon) + 0.15


def test_plan_edge_cases():
    rng = np.random.default_rng(9)
    # P = 1: every token to rank 0, order = identity
    E, k = 8, 2
    p2 = rng.integers(0, E, (64, k)).astype(np.int32)
    p1 = rng.integers(0, E, (64, k)).astype(np.int32)
    F, S, n = O.shuffle_fit(p2, p1, p1, np.zeros(E, np.int32), 1)
    _check_plan(p2, p1, F, S, n, 1.0, 0.9, 1)
    # T = P: one token per rank
    F, S, n = O.shuffle_fit(p2, p1, p1, (np.arange(E) % 4).astype(np.int32), 4)
    _check_plan(p2[:4], p1[:4], F, S, n, 1.0, 0.9, 4)
    # all confidences equal (uniform tables): token order decides, blocks of T/P per rank
    Fu = np.full((E, 4), 0.25, np.float32)
    Su = np.zeros((E, E, 4), np.float32)
    nu = np.zeros((E, E), np.int32)
    owner = _check_plan(p2, p1, Fu, Su, nu, 1.0, 0.9, 4)
    assert np.array_equal(owner, np.arange(64) // 16)
    # k = 1 and few distinct confidences (quantised tables): the sort must keep token order
    q = rng.integers(0, 3, (E, 4)).astype(np.float32) + 1.0
    Fq = (q / q.sum(1, keepdims=True)).astype(np.float32)
    _check_plan(p2[:, :1].copy(), p1[:, :1].copy(), Fq, Su, nu, 1.0, 0.0, 4)


def test_plan_large_and_wide():
    # 65536 tokens (many sort passes with long runs per thread) and P = 64 (a full wave of ranks)
    c, fit, (p2, p1, _) = _trace("ec-top2-p8", 65536, 8192, P=64)
    placement = (np.arange(c.E) % 64).astype(np.int32)
    F, S, n = O.shuffle_fit(*fit, placement, 64)
    _check_plan(p2, p1, F, S, n, 8.0, 0.9, 64)


def test_gpu_fit_feeds_plan():
    # the whole planner on the device: GPU tables, then the plan, equal to the oracle end to end
    c, fit, (p2, p1, cur) = _trace("ec-top6-p8", 2048, 16384)
    grp, _ = O.partition(O.coselect_counts(fit[2], c.E), c.P)
    F, S, n = moe.moe_shuffle_fit(*_d(*fit, grp), c.E, c.P)
    d, conf, owner, order, inverse = moe.moe_shuffle_plan(*_d(p2, p1), F, S, n, 8.0, 0.9)
    F_ref, S_ref, n_ref = O.shuffle_fit(*fit, grp, c.P)
    assert np.array_equal(F.cpu().numpy(), F_ref)
    want = O.shuffle_assign(d.cpu().numpy().astype(np.float64),
                            conf.cpu().numpy().astype(np.float64), c.P)
    assert np.array_equal(owner.cpu().numpy(), want)
