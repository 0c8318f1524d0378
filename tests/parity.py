"""Helpers of the GPU parity tests: expected values from the CPU oracle on the seeded inputs, and
the comparison rules (bit-exact integers; max relative error for floats)."""
from __future__ import annotations

import numpy as np
import torch

from dispatch_expert_gemm_amd import workloads as WL
from oracle import moe_oracle as O

# max relative error bounds per storage dtype (fp32 oracle reference in fp64)
TOL = {"f32": 1e-4, "bf16": 2e-2}


def f64(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        return t.detach().float().cpu().numpy().astype(np.float64)
    return np.asarray(t, dtype=np.float64)


def rel_err(got, ref) -> float:
    """max |got - ref| / max |ref| over the tensor."""
    got, ref = f64(got), f64(ref)
    scale = np.abs(ref).max()
    if scale == 0:
        return float(np.abs(got).max())
    return float(np.abs(got - ref).max() / scale)


def host_inputs(w: WL.Workload) -> dict:
    return dict(x=WL.gen_x(w), logits=WL.gen_logits(w), bias=WL.gen_bias(w))


def placement_for(w: WL.Workload, kind: str, idx=None):
    """contiguous, or the oracle's Algorithm 1 partition of this routing's co-selection."""
    if kind == "contiguous":
        return O.contiguous_placement(w.E, w.W)
    group, _ = O.partition(O.coselect_counts(idx, w.E), w.W)
    return group


def expected_out(w: WL.Workload, x, idx, wts, experts: dict, shared: list, tokens,
                 standin=None, identity=False):
    """out[t] for the listed tokens: sum_j w * FFN_e(x_t) + shared; experts missing from the map
    contribute the stand-in of their slot (one rank's share); identity experts return x_t."""
    x = f64(x)
    tokens = np.asarray(tokens, dtype=np.int64)
    out = np.zeros((len(tokens), x.shape[1]))
    k = idx.shape[1]
    by_e = {}
    for i, t in enumerate(tokens):
        for j in range(k):
            by_e.setdefault(int(idx[t, j]), []).append((i, int(t), j))
    for e, lst in by_e.items():
        ii = np.array([a for a, _, _ in lst])
        tt = np.array([b for _, b, _ in lst])
        jj = np.array([c for _, _, c in lst])
        if identity:
            y = x[tt]
        elif e in experts:
            y = O.swiglu_expert(x[tt], *[f64(m) for m in experts[e]])
        else:
            t0 = w.owned[0]
            y = f64(standin[tt - t0, jj])
        np.add.at(out, ii, wts[tt, jj][:, None].astype(np.float64) * y)
    for s_gu, s_d in shared:
        out += O.swiglu_expert(x[tokens], f64(s_gu), f64(s_d))
    return out
