"""Helpers of the GPU parity tests: expected values from the CPU oracle on the seeded inputs, and
the comparison rules (bit-exact integers; max relative error for floats)."""
from __future__ import annotations

import numpy as np
import torch

from dispatch_expert_gemm_amd import workloads as WL
from oracle import moe_oracle as O

# max relative error bounds per storage dtype (fp32 oracle reference in fp64)
TOL = {"f32": 1e-4, "bf16": 2e-2}

# Element-wise error model of the GPU layer output against the fp64 oracle (every element must
# satisfy |got - ref| <= bound). U is the unit roundoff of the storage type (bf16: 8 significant
# bits, so a rounded value is off by at most 2^-8 of itself).
#  - h rounding: each h_i = silu(g_i) u_i is stored in the storage type, off by a uniformly
#    distributed error of at most U |h_i|; through the down projection Y_n moves by
#    sum_i Wd[n, i] dh_i, a sum of independent terms with standard deviation at most
#    U / sqrt(3) * Q_n, Q_n = sqrt(sum_i Wd[n, i]^2 h_i^2). The weighted terms of one token add
#    in quadrature; LAMBDA standard deviations bound it (8: the largest of 10^9 normal draws is
#    below 6.5).
#  - Y rounding, the dedup partials' rounding and the output's rounding: at most U |value| each,
#    added as is.
#  - fp32 accumulation in both GEMMs (and the gate/up error carried into h): K terms per output,
#    first-order error at most K 2^-24 of the sum of |terms|; the sum of |terms| of the down
#    projection is at most sqrt(I) Q_n (Cauchy-Schwarz). ACC = 2^-16 (bf16, K <= 2^8 MFMA-sized
#    partial sums in sequence) or 2^-13 (fp32 FMA kernel, K <= 2^11 sequential adds) times
#    sqrt(I) Q_n covers it with room for the gate/up error scaled by silu's slope (<= 1.1).
#  - identity experts: out = sum_j w_j x_t in fp32, at most (k + 3) 2^-24 sum_j w_j |x_t|.
# FLOOR: an absolute floor of 1e-6 max|ref| per element.
U = {"f32": 2.0 ** -24, "bf16": 2.0 ** -8}
LAMBDA = 8.0
ACC = {"f32": 2.0 ** -13, "bf16": 2.0 ** -16}
FLOOR = 1e-6


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


def _expert_terms(x, w_gu, w_d, dtype):
    """Oracle rows Y of one expert, the variance bound of the GPU's Y from h rounding, and
    sqrt(I) Q (the Cauchy-Schwarz bound on the down projection's sum of |terms|)."""
    w_gu, w_d = f64(w_gu), f64(w_d)
    y, parts = O.swiglu_expert(x, w_gu, w_d, parts=True)
    h32 = parts["h"].astype(np.float32)
    q2 = ((h32 * h32) @ (w_d.astype(np.float32) ** 2).T).astype(np.float64)
    var = (U[dtype] ** 2 / 3.0) * q2
    acc = np.sqrt(w_d.shape[1]) * np.sqrt(q2)
    return y, var, acc


def expected_out(w: WL.Workload, x, idx, wts, experts: dict, shared: list, tokens,
                 standin=None, identity=False, with_bound=False):
    """out[t] for the listed tokens: sum_j w * FFN_e(x_t) + shared; experts missing from the map
    contribute the stand-in of their slot (one rank's share); identity experts return x_t.
    with_bound: also the element-wise error bound of the GPU output (model above)."""
    x = f64(x)
    tokens = np.asarray(tokens, dtype=np.int64)
    out = np.zeros((len(tokens), x.shape[1]))
    var = np.zeros_like(out) if with_bound else None     # h-rounding variance
    det = np.zeros_like(out) if with_bound else None     # sum of w |Y| (rounded values)
    acc = np.zeros_like(out) if with_bound else None     # accumulation scale
    k = idx.shape[1]
    by_e = {}
    for i, t in enumerate(tokens):
        for j in range(k):
            by_e.setdefault(int(idx[t, j]), []).append((i, int(t), j))
    for e, lst in by_e.items():
        ii = np.array([a for a, _, _ in lst])
        tt = np.array([b for _, b, _ in lst])
        jj = np.array([c for _, _, c in lst])
        wj = wts[tt, jj][:, None].astype(np.float64)
        v = a = None
        if identity:
            y = x[tt]
        elif e in experts:
            if with_bound:
                y, v, a = _expert_terms(x[tt], *experts[e], w.dtype)
            else:
                y = O.swiglu_expert(x[tt], *[f64(m) for m in experts[e]])
        else:
            t0 = w.owned[0]
            y = f64(standin[tt - t0, jj])
        np.add.at(out, ii, wj * y)
        if with_bound:
            np.add.at(det, ii, wj * np.abs(y))
            if v is not None:
                np.add.at(var, ii, wj * wj * v)
                np.add.at(acc, ii, wj * a)
    for s_gu, s_d in shared:
        if with_bound:
            y, v, a = _expert_terms(x[tokens], s_gu, s_d, w.dtype)
            out += y
            det += np.abs(y)
            var += v
            acc += a
        else:
            out += O.swiglu_expert(x[tokens], f64(s_gu), f64(s_d))
    if not with_bound:
        return out
    u = U[w.dtype]
    if identity:
        bound = (k + 3) * 2.0 ** -24 * det
    else:
        # Y rounding (expert rows only, stand-ins are exact), dedup partials, output rounding
        n_round = 2 if w.dedup else 1
        bound = LAMBDA * np.sqrt(var) + n_round * u * det + ACC[w.dtype] * acc
    bound += u * np.abs(out) + FLOOR * np.abs(out).max()
    return out, bound


def elem_ratio(got, ref, bound) -> float:
    """max over elements of |got - ref| / bound (at most 1 passes)."""
    return float((np.abs(f64(got) - f64(ref)) / bound).max())


def expert_rows_with_bound(w: WL.Workload, x, lay: dict, k: int, experts: dict, lo: int,
                           hi: int):
    """Oracle Y for the expert-major rows lo..hi-1 (their experts must be in `experts`) and the
    element-wise bound of the GPU's Y rows (h rounding, Y rounding, accumulation)."""
    x = f64(x)
    tok = lay["slot_of_row"].astype(np.int64) // k
    ref = np.zeros((hi - lo, x.shape[1]))
    bound = np.zeros_like(ref)
    for g, e in enumerate(lay["group_expert"]):
        a, b = max(int(lay["group_offsets"][g]), lo), min(int(lay["group_offsets"][g + 1]), hi)
        if b <= a:
            continue
        y, v, acc = _expert_terms(x[tok[a:b]], *experts[int(e)], w.dtype)
        ref[a - lo:b - lo] = y
        bound[a - lo:b - lo] = LAMBDA * np.sqrt(v) + U[w.dtype] * np.abs(y) + ACC[w.dtype] * acc
    bound += FLOOR * np.abs(ref).max()
    return ref, bound
