"""Pins of the oracle's gate step (CPU only).

Gate = the router's linear layer of FarSkip-Collective section 2.1, G(A) = s(A W_R^T), kept in
FP32 as in Expert Coupling in MoE Pretraining, Appendix A-A1 Table II.
"""
import numpy as np
import torch

from oracle import moe_oracle as O
from dispatch_expert_gemm_amd import workloads as WL


def test_hand_computed_example():
    # two tokens, three experts, small integers: every logit checked by hand
    x = np.array([[1, 2, 3, 4], [0, -1, 2, 0.5]], np.float32)
    w = np.array([[1, 0, 0, 0], [1, 1, 1, 1], [0.5, -1, 0, 2]], np.float32)
    l = O.gate_logits(x, w)
    assert l.dtype == np.float32
    assert l.tolist() == [[1.0, 10.0, 6.5], [0.0, 1.5, 2.0]]


def test_identity_router_selects_coordinates():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 12)).astype(np.float32)
    w = np.zeros((4, 12), np.float32)
    w[np.arange(4), [7, 0, 11, 3]] = 1.0
    np.testing.assert_array_equal(O.gate_logits(x, w), x[:, [7, 0, 11, 3]])


def test_brute_force_loop_tiny():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((3, 6)).astype(np.float32)
    w = rng.standard_normal((5, 6)).astype(np.float32)
    ref = [[float(np.float32(sum(float(x[t, h]) * float(w[e, h]) for h in range(6))))
            for e in range(5)] for t in range(3)]
    np.testing.assert_array_equal(O.gate_logits(x, w), np.array(ref, np.float32))


def test_accumulates_before_rounding():
    # a large cancelling pair: a float32 running sum loses the 1, the exact sum keeps it
    x = np.array([[1e8, 1.0, -1e8]], np.float32)
    w = np.array([[1.0, 1.0, 1.0]], np.float32)
    assert O.gate_logits(x, w)[0, 0] == 1.0


def test_bf16_input_upcast_exactly():
    xb = torch.tensor([[1.0 + 2 ** -7, -3.0]], dtype=torch.bfloat16)
    w = np.array([[1.0, 0.0], [0.0, 1.0]], np.float32)
    l = O.gate_logits(xb.float().numpy(), w)
    assert l[0, 0] == np.float32(1.0 + 2 ** -7) and l[0, 1] == -3.0


def test_router_generator_shape_and_scale():
    w = WL.shrink(WL.WORKLOADS[2])
    r = WL.gen_router(w)
    assert r.shape == (w.E, w.H) and r.dtype == np.float32
    assert abs(float(r.std()) - w.wr_std) < 0.1 * w.wr_std
    np.testing.assert_array_equal(r, WL.gen_router(w))   # seeded
