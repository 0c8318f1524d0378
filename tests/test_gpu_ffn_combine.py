"""GPU parity of the grouped SwiGLU expert FFN, the combine, and the whole layer step against the
CPU oracle (fp64). Floats: max relative error (infinity norm) 1e-4 for fp32, 2e-2 for bf16."""
import numpy as np
import pytest
import torch

from dispatch_expert_gemm_amd import moe
from dispatch_expert_gemm_amd import workloads as WL
from dispatch_expert_gemm_amd.layer import MoELayerRun
from oracle import moe_oracle as O
from tests import parity as P

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda")


def _rand(rng, shape, std, dtype):
    return torch.from_numpy((rng.standard_normal(shape) * std).astype(np.float32)).to(dtype)


SMALL_GROUPS = [0, 1, 127, 128, 300, 64, 0, 129]
LARGE_GROUPS = [1100, 0, 513, 256, 767, 1]          # >= 512 rows per group on average
# 256-row tiles whose group ends 128 rows in (run by half the waves) or 129 rows in (full tile)
TAIL_GROUPS = [384, 129, 640, 0, 1024, 300, 128]


@pytest.mark.parametrize("sizes", [SMALL_GROUPS, LARGE_GROUPS, TAIL_GROUPS],
                         ids=["small", "large", "tails"])
@pytest.mark.parametrize("dtype,H,I", [(torch.bfloat16, 256, 256), (torch.bfloat16, 384, 128),
                                       (torch.float32, 128, 128), (torch.float32, 64, 192)])
@pytest.mark.parametrize("gather", [False, True])
def test_ffn_ragged_groups_and_shared(dtype, H, I, gather, sizes):
    rng = np.random.default_rng(H + I + gather + len(sizes))
    G = len(sizes)
    base = 37                                      # group offsets do not start at zero
    offs = np.concatenate([[0], np.cumsum(sizes)]) + base
    R = int(offs[-1] - base)
    key = "f32" if dtype == torch.float32 else "bf16"
    x = _rand(rng, (R, H), 1.0, dtype)
    if gather:
        # rows come from a shuffled source through the gather map (indexed by absolute row)
        perm = rng.permutation(R)
        src = torch.empty_like(x)
        src[perm] = x
        gmap = np.full(int(offs[-1]), -1, np.int32)
        gmap[base:] = perm + 5
        gbase = torch.tensor([5], dtype=torch.int32, device=DEV)
        rows, gmap_d = src.to(DEV), torch.from_numpy(gmap).to(DEV)
    else:
        rows, gmap_d, gbase = x.to(DEV), None, None
    w_gu = _rand(rng, (G, 2 * I, H), H ** -0.5, dtype)
    w_d = _rand(rng, (G, H, I), I ** -0.5, dtype)
    S, M_sh = 2, 150
    xs = _rand(rng, (M_sh, H), 1.0, dtype)
    s_gu = _rand(rng, (S, 2 * I, H), H ** -0.5, dtype)
    s_d = _rand(rng, (S, H, I), I ** -0.5, dtype)
    h = torch.empty((R, I), dtype=dtype, device=DEV)
    y = torch.full((R, H), float("nan"), dtype=dtype, device=DEV)
    sh_h = torch.empty((S, M_sh, I), dtype=dtype, device=DEV)
    sh_y = torch.full((S, M_sh, H), float("nan"), dtype=dtype, device=DEV)
    offs_d = torch.from_numpy(offs.astype(np.int32)).to(DEV)
    moe.moe_expert_ffn(rows, offs_d, G, w_gu.to(DEV), w_d.to(DEV), h, y, R, row_gather=gmap_d,
                       gather_base=gbase, shared_x=xs.to(DEV), shared_w_gate_up=s_gu.to(DEV),
                       shared_w_down=s_d.to(DEV), shared_h=sh_h, shared_y=sh_y)
    torch.cuda.synchronize()
    ref = np.zeros((R, H))
    for g in range(G):
        lo, hi = offs[g] - base, offs[g + 1] - base
        if hi > lo:
            ref[lo:hi] = O.swiglu_expert(P.f64(x[lo:hi]), P.f64(w_gu[g]), P.f64(w_d[g]))
    assert P.rel_err(y.cpu(), ref) <= P.TOL[key]
    for s in range(S):
        rs = O.swiglu_expert(P.f64(xs), P.f64(s_gu[s]), P.f64(s_d[s]))
        assert P.rel_err(sh_y[s].cpu(), rs) <= P.TOL[key]


@pytest.mark.parametrize("mean_rows", [3, 300], ids=["128-row-tiles", "256-row-tiles"])
def test_ffn_most_groups_and_shared_experts(mean_rows):
    """The largest group counts the GEMM takes: MOE_MAX_EXPERTS routed groups plus 16 shared
    experts, so the device-side prefix of row tiles spans 528 groups in several wave passes and
    the tile decode searches all of them; a few rows per group (128-row tiles) or a few hundred
    (256-row tiles, many of them half tiles)."""
    dtype = torch.bfloat16
    rng = np.random.default_rng(mean_rows)
    G, S, M_sh, H, I = 512, 16, 40, 128, 128
    sizes = rng.integers(0, 2 * mean_rows + 1, size=G)
    offs = np.concatenate([[0], np.cumsum(sizes)])
    R = int(offs[-1])
    x = _rand(rng, (R, H), 1.0, dtype)
    w_gu = _rand(rng, (G, 2 * I, H), H ** -0.5, dtype)
    w_d = _rand(rng, (G, H, I), I ** -0.5, dtype)
    xs = _rand(rng, (M_sh, H), 1.0, dtype)
    s_gu = _rand(rng, (S, 2 * I, H), H ** -0.5, dtype)
    s_d = _rand(rng, (S, H, I), I ** -0.5, dtype)
    h = torch.empty((R, I), dtype=dtype, device=DEV)
    y = torch.full((R, H), float("nan"), dtype=dtype, device=DEV)
    sh_h = torch.empty((S, M_sh, I), dtype=dtype, device=DEV)
    sh_y = torch.full((S, M_sh, H), float("nan"), dtype=dtype, device=DEV)
    offs_d = torch.from_numpy(offs.astype(np.int32)).to(DEV)
    moe.moe_expert_ffn(x.to(DEV), offs_d, G, w_gu.to(DEV), w_d.to(DEV), h, y, R,
                       shared_x=xs.to(DEV), shared_w_gate_up=s_gu.to(DEV),
                       shared_w_down=s_d.to(DEV), shared_h=sh_h, shared_y=sh_y)
    torch.cuda.synchronize()
    ref = np.zeros((R, H))
    xf, gu, d = P.f64(x), P.f64(w_gu), P.f64(w_d)
    for g in range(G):
        lo, hi = offs[g], offs[g + 1]
        if hi > lo:
            ref[lo:hi] = O.swiglu_expert(xf[lo:hi], gu[g], d[g])
    assert P.rel_err(y.cpu(), ref) <= P.TOL["bf16"]
    xsf = P.f64(xs)
    for s_ in range(S):
        rs = O.swiglu_expert(xsf, P.f64(s_gu[s_]), P.f64(s_d[s_]))
        assert P.rel_err(sh_y[s_].cpu(), rs) <= P.TOL["bf16"]


def test_ffn_no_rows_and_shared_only():
    dtype = torch.bfloat16
    rng = np.random.default_rng(9)
    H, I, G = 128, 128, 3
    offs = torch.zeros(G + 1, dtype=torch.int32, device=DEV)
    w_gu = _rand(rng, (G, 2 * I, H), 0.1, dtype).to(DEV)
    w_d = _rand(rng, (G, H, I), 0.1, dtype).to(DEV)
    h = torch.empty((8, I), dtype=dtype, device=DEV)
    y = torch.full((8, H), 7.0, dtype=dtype, device=DEV)
    moe.moe_expert_ffn(torch.empty((8, H), dtype=dtype, device=DEV), offs, G, w_gu, w_d, h, y, 8)
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)                   # nothing to compute, nothing written
    xs = _rand(rng, (33, H), 1.0, dtype)
    s_gu = _rand(rng, (1, 2 * I, H), 0.1, dtype)
    s_d = _rand(rng, (1, H, I), 0.1, dtype)
    sh_h = torch.empty((1, 33, I), dtype=dtype, device=DEV)
    sh_y = torch.empty((1, 33, H), dtype=dtype, device=DEV)
    moe.moe_expert_ffn(None, None, 0, None, None, None, None, 0, shared_x=xs.to(DEV),
                       shared_w_gate_up=s_gu.to(DEV), shared_w_down=s_d.to(DEV), shared_h=sh_h,
                       shared_y=sh_y)
    torch.cuda.synchronize()
    ref = O.swiglu_expert(P.f64(xs), P.f64(s_gu[0]), P.f64(s_d[0]))
    assert P.rel_err(sh_y[0].cpu(), ref) <= P.TOL["bf16"]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_combine_flat_and_dedup(dtype):
    rng = np.random.default_rng(3)
    N, E, k, W, H = 96, 12, 3, 4, 64
    key = "f32" if dtype == torch.float32 else "bf16"
    idx = np.argsort(rng.random((N, E)), axis=1)[:, :k].astype(np.int32)
    wts = rng.random((N, k)).astype(np.float32)
    pi = O.contiguous_placement(E, W)[rng.permutation(E)]
    ref_lay = O.layout(idx, pi, W)
    y = _rand(rng, (N * k, H), 1.0, dtype)
    sh = _rand(rng, (2, N, H), 1.0, dtype)
    lay = moe.Layout(N, E, k, W, H)
    idx_d, w_d, pi_d = (torch.from_numpy(a).to(DEV) for a in (idx, wts, pi.astype(np.int32)))
    moe.moe_dispatch_layout(lay, idx_d, pi_d)
    out = torch.empty((N, H), dtype=dtype, device=DEV)
    moe.moe_combine(lay, y.to(DEV), idx_d, w_d, out, expert_rank=pi_d, shared=sh.to(DEV))
    torch.cuda.synchronize()
    ref = O.combine_a2a(P.f64(y), ref_lay, wts, shared=P.f64(sh))
    assert P.rel_err(out.cpu(), ref) <= P.TOL[key]
    # owned slice
    out2 = torch.empty((20, H), dtype=dtype, device=DEV)
    moe.moe_combine(lay, y.to(DEV), idx_d, w_d, out2, expert_rank=pi_d, t_begin=40, t_end=60)
    torch.cuda.synchronize()
    assert P.rel_err(out2.cpu(), O.combine_a2a(P.f64(y), ref_lay, wts, 40, 60)) <= P.TOL[key]
    # dedup: expert-rank partials, then the owner sum
    part = torch.empty((N * min(k, W), H), dtype=dtype, device=DEV)
    out3 = torch.empty((N, H), dtype=dtype, device=DEV)
    moe.moe_combine(lay, y.to(DEV), idx_d, w_d, out3, expert_rank=pi_d, dedup=True, partial=part,
                    shared=sh.to(DEV))
    torch.cuda.synchronize()
    rp = O.dedup_partials(P.f64(y), ref_lay, idx, wts, pi)
    assert P.rel_err(part[:ref_lay["D"]].cpu(), rp) <= P.TOL[key]
    assert P.rel_err(out3.cpu(), O.combine_dedup(rp, ref_lay, k, shared=P.f64(sh))) <= P.TOL[key]


def _shrunk(cfg):
    w = WL.WORKLOADS[cfg]
    if cfg == 1:
        return w
    if cfg == 2:
        return WL.shrink(w, N=512, H=256, E=16, k=6, W=8, I=256)
    if cfg == 3:
        return WL.shrink(w, N=1024, H=256, E=32, k=8, W=8, I=256)
    if cfg == 4:
        return WL.shrink(w, N=512, H=256, E=16, k=1, W=4, I=384)
    return WL.shrink(w, N=2048, H=256)


def _check_step(w, placement=None, tokens=None, sync_standins=True, bound=False):
    """One layer step on the GPU against the oracle: max relative error within the dtype's
    tolerance and, with bound=True, every element within the element-wise error model."""
    run = MoELayerRun(w, placement=placement)
    run.route()
    run.dispatch()
    if w.dst_rank >= 0 and sync_standins:
        run.place_standins()
    run.ffn()
    run.combine()
    torch.cuda.synchronize()
    x = WL.gen_x(w)
    idx, wts = O.route(WL.gen_logits(w), WL.gen_bias(w), w.k, w.gate)
    experts, shared = {}, []
    if w.expert == "swiglu":
        wgu, wd = run.host["experts"]
        experts = {e: (wgu[i], wd[i]) for i, e in enumerate(run.local)}
        shared = [WL.gen_shared(w, s) for s in range(w.n_shared)]
    t0, t1 = w.owned
    tokens = np.arange(t0, t1) if tokens is None else np.asarray(tokens)
    standin = WL.gen_standin(w) if w.dst_rank >= 0 else None
    res = P.expected_out(w, x, idx, wts, experts, shared, tokens, standin=standin,
                         identity=w.expert == "identity", with_bound=bound)
    ref, bnd = res if bound else (res, None)
    got = run.out.cpu()[tokens - t0]
    err = P.rel_err(got, ref)
    assert err <= P.TOL[w.dtype], err
    ratio = None
    if bound:
        ratio = P.elem_ratio(got, ref, bnd)
        assert ratio <= 1.0, f"element-wise error {ratio:.3f} of the bound"
    return run, err, ratio


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_step_shrunk_workloads(cfg):
    _check_step(_shrunk(cfg), bound=True)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_step_shrunk_dedup_variants(cfg):
    w = _shrunk(cfg)
    _check_step(w.replace(dedup=not w.dedup), bound=True)


def test_step_correlated_placement_identity():
    w = _shrunk(5)
    idx = O.route(WL.gen_logits(w), None, w.k, w.gate)[0]
    pi = P.placement_for(w, "correlated", idx)
    for dedup in (True, False):
        _check_step(w.replace(dedup=dedup), placement=pi, bound=True)


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_step_full_workloads_every_token(cfg):
    # every owned token of the full workload against the oracle: the max relative error within
    # the dtype's tolerance and every element within the element-wise error model
    w = WL.WORKLOADS[cfg]
    print(f"[full {w.name}] start", flush=True)
    run, err, ratio = _check_step(w, bound=True)
    t0, t1 = w.owned
    print(f"[full {w.name}] {t1 - t0} tokens: max relative error {err:.3e}, element-wise "
          f"error at most {ratio:.3f} of the bound", flush=True)
    # bit-identical on a second pass
    first = run.out.clone()
    run.step()
    torch.cuda.synchronize()
    assert torch.equal(_bits(first), _bits(run.out))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_step_from_x_full_workloads_every_token(cfg):
    # the step as the benchmark times these workloads: the router linear layer on the device,
    # its route and count rows, dispatch, expert FFN and combine. The selection must equal the
    # oracle's route on the device's logits (their fp32 rounding decides near ties), and every
    # owned token must match the oracle's layer on that routing, element-wise.
    w = WL.WORKLOADS[cfg]
    print(f"[full from x {w.name}] start", flush=True)
    run = MoELayerRun(w)
    run.gate_route()
    run.dispatch()
    if w.dst_rank >= 0:
        run.place_standins()
    run.ffn()
    run.combine()
    torch.cuda.synchronize()
    idx, wts = O.route(run.gate_logits.cpu().numpy(), WL.gen_bias(w), w.k, w.gate)
    assert np.array_equal(run.topk_idx.cpu().numpy(), idx)
    assert (np.abs(run.topk_w.cpu().numpy().astype(np.float64) - wts) / np.abs(wts)).max() <= 1e-4
    experts, shared = {}, []
    if w.expert == "swiglu":
        wgu, wd = run.host["experts"]
        experts = {e: (wgu[i], wd[i]) for i, e in enumerate(run.local)}
        shared = [WL.gen_shared(w, s) for s in range(w.n_shared)]
    t0, t1 = w.owned
    tokens = np.arange(t0, t1)
    standin = WL.gen_standin(w) if w.dst_rank >= 0 else None
    ref, bnd = P.expected_out(w, WL.gen_x(w), idx, wts, experts, shared, tokens,
                              standin=standin, identity=w.expert == "identity", with_bound=True)
    got = run.out.cpu()[tokens - t0]
    err = P.rel_err(got, ref)
    assert err <= P.TOL[w.dtype], err
    ratio = P.elem_ratio(got, ref, bnd)
    assert ratio <= 1.0, f"element-wise error {ratio:.3f} of the bound"
    print(f"[full from x {w.name}] {t1 - t0} tokens: max relative error {err:.3e}, "
          f"element-wise error at most {ratio:.3f} of the bound", flush=True)


@pytest.mark.timeout(900)
def test_full_workload3_every_expert_row():
    # one EP8 rank's share: every row the rank's grouped GEMM computes (all tokens routed to
    # its 32 experts, not only the owned ones) against the oracle, element-wise
    w = WL.WORKLOADS[3]
    print(f"[full {w.name} rows] start", flush=True)
    run = MoELayerRun(w)
    run.route()
    run.dispatch()
    run.ffn()
    torch.cuda.synchronize()
    idx, _ = O.route(WL.gen_logits(w), WL.gen_bias(w), w.k, w.gate)
    lay = O.layout(idx, O.contiguous_placement(w.E, w.W), w.W)
    lo, hi = int(lay["rank_offsets"][0]), int(lay["rank_offsets"][1])
    wgu, wd = run.host["experts"]
    experts = {e: (wgu[i], wd[i]) for i, e in enumerate(run.local)}
    ref, bnd = P.expert_rows_with_bound(w, WL.gen_x(w), lay, w.k, experts, lo, hi)
    got = run.y[lo:hi].cpu()
    err, ratio = P.rel_err(got, ref), P.elem_ratio(got, ref, bnd)
    print(f"[full {w.name} rows] {hi - lo} rows: max relative error {err:.3e}, element-wise "
          f"{ratio:.3f} of the bound", flush=True)
    assert err <= P.TOL[w.dtype] and ratio <= 1.0


@pytest.mark.timeout(900)
def test_full_workload3_dedup_every_token():
    # the same rank's share with the deduplicating dispatcher: one pair row per (token, rank),
    # the GEMM expands them through the gather map, the other ranks' partials are stand-ins
    w = WL.WORKLOADS[3].replace(dedup=True)
    print(f"[full {w.name} dedup] start", flush=True)
    run, err, ratio = _check_step(w, bound=True)
    print(f"[full {w.name} dedup] max relative error {err:.3e}, element-wise {ratio:.3f} of "
          f"the bound", flush=True)


@pytest.mark.parametrize("dedup", [False, True])
@pytest.mark.parametrize("dst_rank", [0, 3])
def test_step_one_rank_share(dst_rank, dedup):
    # one rank's share of a shrunk DeepSeek-V3-shaped layer, for a rank whose partition does
    # not start at row 0 (its outputs land in place with no host read of the rank's offset)
    w = WL.shrink(WL.WORKLOADS[3], N=1024, H=256, E=32, k=8, W=8, I=256, dst_rank=dst_rank)
    _check_step(w.replace(dedup=dedup), bound=True)


@pytest.mark.timeout(900)
def test_step_full_workload5_correlated_placement_every_token():
    # the correlated-routing workload at full size under the placement Algorithm 1 computes
    # from its own routing (dedup dispatch and combine through the pair rows)
    w = WL.WORKLOADS[5]
    idx = O.route(WL.gen_logits(w), None, w.k, w.gate)[0]
    pi = P.placement_for(w, "correlated", idx)
    print(f"[full {w.name} correlated] start", flush=True)
    _, err, ratio = _check_step(w, placement=pi, bound=True)
    print(f"[full {w.name} correlated] max relative error {err:.3e}, element-wise "
          f"{ratio:.3f} of the bound", flush=True)
