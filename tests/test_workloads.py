"""The seeded input generators: reproducible, with the stated shapes, scales and structure."""
import math

import numpy as np
import torch

from dispatch_expert_gemm_amd import workloads as WL
from oracle import moe_oracle as O


def test_reproducible_and_independent_streams():
    w = WL.shrink(WL.WORKLOADS[2], N=64, H=128, I=64, E=8, k=2, W=4)
    assert torch.equal(WL.gen_x(w), WL.gen_x(w))
    a = WL.gen_expert(w, 3)
    b = WL.gen_expert(w, 3)
    c = WL.gen_expert(w, 4)
    assert torch.equal(a[0], b[0]) and not torch.equal(a[0], c[0])
    g_gu, g_d = WL.gen_experts(w, [4, 3])
    assert torch.equal(g_gu[1], a[0]) and torch.equal(g_d[0], c[1])


def test_scales():
    w = WL.WORKLOADS[2]
    l = WL.gen_logits(w)
    assert l.dtype == np.float32 and l.shape == (w.N, w.E)
    assert abs(l.std() - 0.02 * math.sqrt(w.H)) < 0.02
    assert abs(WL.gen_bias(w).std() - 0.5) < 0.15
    small = WL.shrink(w, N=256, H=256, I=128, E=4)
    assert abs(WL.gen_expert(small, 0)[0].float().std().item() - 1 / 16) < 0.003


def test_bf16_is_round_to_nearest_even():
    w = WL.shrink(WL.WORKLOADS[2], N=8, H=64)
    x = WL.gen_x(w)
    assert x.dtype == torch.bfloat16
    # regenerate the fp32 draws and round by hand: ties to the even mantissa
    f = (WL._rng(w.seed, WL._S_X).standard_normal((w.N, w.H), np.float32) * w.x_std)
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    assert np.array_equal(x.view(torch.int16).numpy().view(np.uint16), r)


def test_hot_pair_share_of_correlated_workload():
    """About 42% of tokens draw one of the 0.8% hot pairs; others hit one only by chance."""
    w = WL.WORKLOADS[5]
    pairs, token_pair = WL.hot_pair_structure(w)
    assert len(pairs) == 16 and len(set(pairs.reshape(-1).tolist())) == 32
    idx, _ = O.route(WL.gen_logits(w), None, w.k, "softmax")
    hot = {frozenset(p) for p in pairs.tolist()}
    share = np.mean([frozenset(r) in hot for r in idx.tolist()])
    null = 16 / (w.E * (w.E - 1) // 2)
    assert abs(share - (0.42 + 0.58 * null)) < 0.01
    # without the planted boost the share falls to the independence null
    plain = WL.gen_logits(w.replace(hot_pairs=False))
    share0 = np.mean([frozenset(r) in hot for r in O.route(plain, None, 2, "softmax")[0].tolist()])
    assert abs(share0 - null) < 0.004
    # Zipf(1.1) popularity: the most popular pair is the most frequent
    counts = np.bincount(token_pair[token_pair >= 0], minlength=16)
    assert counts.argmax() == 0 and counts[0] > counts[-1] * 15


def test_standin_shape():
    w = WL.shrink(WL.WORKLOADS[3], N=64, H=32, E=16, k=4, W=8, I=32)
    s = WL.gen_standin(w)
    assert s.shape == (w.owned[1] - w.owned[0], w.k, w.H) and w.owned == (0, 8)
