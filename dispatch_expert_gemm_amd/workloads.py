"""The five synthetic MoE-layer workloads and their seeded input generators.

This module is shared by the HIP path's harness and by the CPU oracle's tests. It holds no
arithmetic of the layer: only the workload shapes, random draws, rounding of the draws to the
storage dtype, and the hot-pair structure that the correlated-routing workload plants in its
router logits.

Every tensor comes from its own named substream ``SeedSequence([seed, stream, sub])`` so that
any part (one expert's weights, say) can be regenerated alone.

Router logits are generated directly, not as ``x @ W_R^T``: the layer's route step starts from
the router's fp32 output (FarSkip-Collective, section 2.1 "Expert Parallelism": the gate is a linear
layer followed by a sparse selection, and only the selection is on this path). With
``x ~ N(0, 1)`` and ``W_R ~ N(0, s)`` each entry of ``x W_R^T`` is a sum of H products of
variance ``s^2``, so the logits are drawn as ``N(0, s * sqrt(H))``.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

# substream ids
_S_X, _S_LOGITS, _S_BIAS, _S_HOT, _S_STANDIN, _S_EXPERT, _S_SHARED = 1, 2, 3, 4, 5, 6, 7
_S_ROUTER = 8


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    N: int            # tokens
    H: int            # hidden width
    E: int            # routed experts
    k: int            # experts per token
    W: int            # simulated expert-parallel ranks
    I: int            # expert intermediate width (0 for identity experts)
    n_shared: int     # always-on shared experts (same shape as a routed expert)
    dtype: str        # "f32" | "bf16": storage type of x, weights, rows, outputs
    gate: str         # "softmax" (top-k, renormalised) | "sigmoid"
    expert: str       # "swiglu" | "identity"
    x_std: float
    wr_std: float     # router weight std (sets the logit scale)
    w_std: float      # expert / shared weight std
    bias_std: float   # per-expert router bias std; 0 = no bias
    hot_pairs: bool   # plant co-selected expert pairs in the logits
    dst_rank: int     # -1: every rank's share on this GPU; r: permute / GEMM only for rank r
    owned: tuple      # (t_begin, t_end) tokens whose combine runs here
    dedup: bool       # dispatch one row per (token, rank) instead of one per (token, expert)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def elt_bytes(self):
        return 4 if self.dtype == "f32" else 2

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _w(**kw):
    base = dict(n_shared=0, x_std=1.0, wr_std=0.02, bias_std=0.0, hot_pairs=False,
                dst_rank=-1, owned=None, dedup=False, expert="swiglu", gate="softmax")
    base.update(kw)
    if base["owned"] is None:
        base["owned"] = (0, base["N"])
    return Workload(**base)


WORKLOADS = {
    1: _w(name="tiny-fp32", seed=1, N=64, H=128, E=8, k=2, W=4, I=256, dtype="f32",
          w_std=0.02),
    2: _w(name="dsv2-lite-bf16", seed=2, N=4096, H=2048, E=64, k=6, W=8, I=1408, n_shared=2,
          dtype="bf16", w_std=1.0 / math.sqrt(2048), bias_std=0.5),
    3: _w(name="dsv3-ep8-rank0-bf16", seed=3, N=16384, H=7168, E=256, k=8, W=8, I=2048,
          dtype="bf16", w_std=1.0 / math.sqrt(7168), bias_std=0.5, dst_rank=0,
          owned=(0, 2048)),
    4: _w(name="llama4-scout-bf16", seed=4, N=8192, H=5120, E=16, k=1, W=4, I=8192,
          n_shared=1, dtype="bf16", gate="sigmoid", w_std=1.0 / math.sqrt(5120),
          bias_std=0.5),
    5: _w(name="corr-routing-fp32", seed=5, N=32768, H=2048, E=64, k=2, W=32, I=0,
          dtype="f32", expert="identity", w_std=0.0, hot_pairs=True, dedup=True),
}


def shrink(w: Workload, **kw) -> Workload:
    """A smaller workload of the same structure (for parity runs the oracle finishes quickly).

    Keeps the weight std tied to the new H where the full workload ties it to H.
    """
    new = dataclasses.replace(w, **kw)
    if w.w_std and abs(w.w_std - 1.0 / math.sqrt(w.H)) < 1e-12:
        new = dataclasses.replace(new, w_std=1.0 / math.sqrt(new.H))
    if "owned" not in kw:
        if w.owned == (0, w.N):
            new = dataclasses.replace(new, owned=(0, new.N))
        else:  # the owner slice of rank dst_rank
            per = new.N // new.W
            r = max(new.dst_rank, 0)
            new = dataclasses.replace(new, owned=(r * per, (r + 1) * per))
    return new


def _rng(seed: int, stream: int, sub: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream, sub])))


def _store(a: np.ndarray, dtype: str) -> torch.Tensor:
    """fp32 draws to the storage dtype (bf16 by round-to-nearest-even)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t if dtype == "f32" else t.to(torch.bfloat16)


def gen_x(w: Workload) -> torch.Tensor:
    """Hidden states [N, H] ~ N(0, x_std), storage dtype."""
    return _store(_rng(w.seed, _S_X).standard_normal((w.N, w.H), np.float32) * w.x_std,
                  w.dtype)


def gen_bias(w: Workload):
    """Per-expert router bias [E] f32 ~ N(0, bias_std), or None."""
    if not w.bias_std:
        return None
    return (_rng(w.seed, _S_BIAS).standard_normal(w.E, np.float32) * w.bias_std).astype(
        np.float32)


def hot_pair_structure(w: Workload):
    """The planted co-selection of the correlated-routing workload.

    About 0.8% of the E(E-1)/2 expert pairs are hot: floor(0.008 * E(E-1)/2) disjoint pairs
    taken from a seeded permutation of the experts. Each token, with probability 0.42, draws one
    hot pair with Zipf(1.1) popularity over the pair ranks and gets +10 on both logits; the
    others keep their plain logits (Expert Coupling in MoE Pretraining, section II-B: 0.8% of
    pairs carry 42% of tokens at top-2).

    Returns (pairs [P, 2] int64, token_pair [N] int64 with -1 for tokens without a hot pair).
    """
    r = _rng(w.seed, _S_HOT)
    n_hot = int(0.008 * w.E * (w.E - 1) // 2)
    perm = r.permutation(w.E)
    pairs = perm[: 2 * n_hot].reshape(n_hot, 2).astype(np.int64)
    pop = np.arange(1, n_hot + 1, dtype=np.float64) ** -1.1
    pop /= pop.sum()
    has = r.random(w.N) < 0.42
    which = r.choice(n_hot, size=w.N, p=pop)
    token_pair = np.where(has, which, -1).astype(np.int64)
    return pairs, token_pair


HOT_BOOST = 10.0


def gen_logits(w: Workload) -> np.ndarray:
    """Router logits [N, E] f32 ~ N(0, wr_std * sqrt(H) * x_std), plus the hot-pair boost."""
    std = w.wr_std * math.sqrt(w.H) * w.x_std
    l = _rng(w.seed, _S_LOGITS).standard_normal((w.N, w.E), np.float32) * np.float32(std)
    l = l.astype(np.float32)
    if w.hot_pairs:
        pairs, token_pair = hot_pair_structure(w)
        t = np.nonzero(token_pair >= 0)[0]
        for c in (0, 1):
            l[t, pairs[token_pair[t], c]] += np.float32(HOT_BOOST)
    return l


def gen_router(w: Workload) -> np.ndarray:
    """Router (gate) weights W_R [E, H] f32 ~ N(0, wr_std); the gate stays fp32 in every
    configuration (Expert Coupling in MoE Pretraining, Appendix A-A1 Table II: FP32 linear gate).
    Used by the fused gate path, whose logits are x W_R^T."""
    return (_rng(w.seed, _S_ROUTER).standard_normal((w.E, w.H), np.float32) *
            np.float32(w.wr_std)).astype(np.float32)


def _expert_weights(seed, stream, sub, I, H, std, dtype):
    r = _rng(seed, stream, sub)
    w_gu = r.standard_normal((2 * I, H), np.float32) * np.float32(std)
    w_d = r.standard_normal((H, I), np.float32) * np.float32(std)
    return _store(w_gu, dtype), _store(w_d, dtype)


def gen_expert(w: Workload, e: int):
    """Routed expert e: (w_gu [2I, H] = [gate rows; up rows], w_d [H, I]), storage dtype."""
    return _expert_weights(w.seed, _S_EXPERT, e, w.I, w.H, w.w_std, w.dtype)


def gen_shared(w: Workload, s: int):
    """Shared expert s, same shapes as a routed expert."""
    return _expert_weights(w.seed, _S_SHARED, s, w.I, w.H, w.w_std, w.dtype)


def gen_experts(w: Workload, experts, threads: int = 8):
    """Stacked weights of the listed experts: (w_gu [G, 2I, H], w_d [G, H, I])."""
    experts = list(experts)
    G = len(experts)
    w_gu = torch.empty((G, 2 * w.I, w.H), dtype=w.torch_dtype)
    w_d = torch.empty((G, w.H, w.I), dtype=w.torch_dtype)

    def one(i):
        a, b = gen_expert(w, experts[i])
        w_gu[i].copy_(a)
        w_d[i].copy_(b)

    with ThreadPoolExecutor(max(1, threads)) as ex:
        list(ex.map(one, range(G)))
    return w_gu, w_d


def gen_shared_all(w: Workload):
    """Stacked shared-expert weights (w_gu [S, 2I, H], w_d [S, H, I]), or (None, None)."""
    if w.n_shared == 0:
        return None, None
    parts = [gen_shared(w, s) for s in range(w.n_shared)]
    return (torch.stack([p[0] for p in parts]), torch.stack([p[1] for p in parts]))


def gen_standin(w: Workload) -> torch.Tensor:
    """Stand-in outputs [t_end - t_begin, k, H] ~ N(0, 1) of the experts on other ranks.

    When only one rank's experts run here, the owned tokens' slots routed to experts of other
    ranks take these values as the rows those ranks would return in the combine.
    """
    t0, t1 = w.owned
    a = _rng(w.seed, _S_STANDIN).standard_normal((t1 - t0, w.k, w.H), np.float32)
    return _store(a, w.dtype)


# ----------------------------------------------------------------------------------------------
# routing traces for the token-shuffle planner
# ----------------------------------------------------------------------------------------------
_S_SHUF_MODEL, _S_SHUF_TOKENS = 20, 21


@dataclasses.dataclass(frozen=True)
class ShuffleTrace:
    """Synthetic routing of T tokens at three consecutive MoE positions (m-2, m-1, m).

    Stand-in for the routing traces of a trained model (Expert Coupling in MoE Pretraining,
    section V-B; section II-B: experts chosen at one layer predict those of the next). Each token
    has a latent class; at every position each class prefers its own `pref` experts, and each of
    a token's k slots comes from its class's preferred set with probability about `rho`, from all
    E experts otherwise (k distinct experts, weighted sampling without replacement). The class
    persists across positions, which makes the routing correlated across layers and within one.
    """
    name: str
    seed: int
    T: int          # tokens of one plan (the sequence shard group of TP = EP = P ranks)
    E: int
    k: int
    P: int          # ranks (TP = EP = P)
    classes: int
    pref: int       # preferred experts per class and position
    rho: float
    fit_tokens: int  # tokens of the separate trace the tables are fit on


SHUFFLE_TRACES = {
    # 128 experts, top-2 / top-6, TP8 EP8 and TP16 EP16 (section VI: 12-layer models with 128
    # experts; sequence length 8192). 16 classes of 8 preferred experts with rho = 0.8 give,
    # under correlated placement, locality of the same order as section VI-C reports
    "ec-top2-p8": ShuffleTrace("ec-top2-p8", 71, 8192, 128, 2, 8, 16, 8, 0.8, 65536),
    "ec-top6-p8": ShuffleTrace("ec-top6-p8", 72, 8192, 128, 6, 8, 16, 8, 0.8, 65536),
    "ec-top6-p16": ShuffleTrace("ec-top6-p16", 73, 8192, 128, 6, 16, 16, 8, 0.8, 65536),
}


def shuffle_class_sets(c: ShuffleTrace) -> np.ndarray:
    """Preferred experts [3, classes, pref] int64 of every class at positions m-2, m-1, m."""
    r = _rng(c.seed, _S_SHUF_MODEL)
    return np.stack([np.stack([r.choice(c.E, size=c.pref, replace=False)
                               for _ in range(c.classes)]) for _ in range(3)])


def gen_shuffle_trace(c: ShuffleTrace, split: str = "eval"):
    """Top-k expert sets of one trace at positions m-2, m-1, m: three int32 arrays [n, k].

    split "eval": the T tokens of the plan; "fit": fit_tokens other tokens of the same model (the
    offline trace the tables come from). Sampling without replacement is done by adding Gumbel
    noise to the log weights and keeping the k largest.
    """
    n = c.T if split == "eval" else c.fit_tokens
    sub = 0 if split == "eval" else 1
    r = _rng(c.seed, _S_SHUF_TOKENS, sub)
    sets = shuffle_class_sets(c)
    cls = r.integers(0, c.classes, size=n)
    out = []
    for pos in range(3):
        wgt = np.full((n, c.E), (1.0 - c.rho) / c.E)
        rows = np.repeat(np.arange(n), c.pref)
        wgt[rows, sets[pos][cls].ravel()] += c.rho / c.pref
        score = np.log(wgt) + r.gumbel(size=(n, c.E))
        top = np.argpartition(-score, c.k - 1, axis=1)[:, : c.k]
        order = np.argsort(-np.take_along_axis(score, top, axis=1), axis=1, kind="stable")
        out.append(np.take_along_axis(top, order, axis=1).astype(np.int32))
    return out[0], out[1], out[2]
