"""GPU parity of route, dispatch layout (+ dedup) and permute against the CPU oracle.

Integers (expert ids, counts, offsets, permutations, pair rows, send matrices) and the permuted
rows (a pure copy) must be bit-exact; routing weights within 1e-4 relative."""
import numpy as np
import pytest
import torch

from dispatch_expert_gemm_amd import moe
from dispatch_expert_gemm_amd import workloads as WL
from oracle import moe_oracle as O
from tests import parity as P

pytestmark = pytest.mark.gpu

INT_FIELDS = ("expert_counts", "expert_offsets", "group_expert", "group_offsets", "rank_counts",
              "rank_offsets", "send_counts", "row_of_slot", "slot_of_row", "pair_counts",
              "pair_offsets", "pair_of_slot", "pair_send_counts", "expand_src")


def _route_check(logits, bias, k, gate):
    dev = torch.device("cuda")
    lg = torch.from_numpy(np.ascontiguousarray(logits, np.float32)).to(dev)
    b = None if bias is None else torch.from_numpy(np.asarray(bias, np.float32)).to(dev)
    idx, w = moe.moe_route(lg, b, k, gate)
    torch.cuda.synchronize()
    ridx, rw = O.route(logits, bias, k, gate)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    rel = np.abs(w.cpu().numpy().astype(np.float64) - rw) / np.abs(rw)
    assert rel.max() <= 1e-4
    return ridx


def _layout_check(idx_host, placement, W, H=8, x=None, dedup=False, dst_rank=-1, E=None):
    N, k = idx_host.shape
    E = len(placement) if placement is not None else E
    dev = torch.device("cuda")
    idx = torch.from_numpy(np.ascontiguousarray(idx_host, np.int32)).to(dev)
    pl = None if placement is None else torch.from_numpy(np.asarray(placement, np.int32)).to(dev)
    lay = moe.Layout(N, E, k, W, H)
    rows = None
    if x is not None:
        kw = min(k, W)
        cap = (N * kw if dedup else N * k) if dst_rank < 0 else (N if dedup else N * min(k, E // W))
        rows = torch.full((cap, H), float("nan"), dtype=x.dtype, device=dev)
    moe.moe_dispatch_layout(lay, idx, pl, None if x is None else x.to(dev), dedup=dedup,
                            dst_rank=dst_rank, rows_out=rows)
    torch.cuda.synchronize()
    pi = placement if placement is not None else O.contiguous_placement(E, W)
    ref = O.layout(idx_host, pi, W)
    for f in INT_FIELDS:
        got = lay[f].cpu().numpy()
        assert np.array_equal(got, ref[f].reshape(-1)), f
    D = ref["D"]
    assert np.array_equal(lay["pair_token"].cpu().numpy()[:D], ref["pair_token"])
    if x is not None:
        want = O.dispatch_rows(x.float().numpy() if x.dtype == torch.bfloat16 else x.numpy(),
                               ref, dedup, dst_rank)
        got = rows[:want.shape[0]].cpu()
        # a pure copy: compare the stored bits
        wantt = torch.from_numpy(np.ascontiguousarray(want)).to(x.dtype)
        assert torch.equal(got.view(torch.int16) if x.dtype == torch.bfloat16 else got.view(torch.int32),
                           wantt.view(torch.int16) if x.dtype == torch.bfloat16 else wantt.view(torch.int32))
    return lay, ref


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_route_full_workloads(cfg):
    w = WL.WORKLOADS[cfg]
    _route_check(WL.gen_logits(w), WL.gen_bias(w), w.k, w.gate)


def test_route_ties_and_edges():
    rng = np.random.default_rng(0)
    # heavy ties: integer logits
    for E, k in [(8, 2), (64, 6), (256, 8), (16, 16), (1, 1), (3, 2), (100, 7), (512, 64),
                 (512, 8), (33, 1)]:
        l = rng.integers(-2, 3, size=(300, E)).astype(np.float32)
        _route_check(l, None, k, "softmax")
        _route_check(l * 0.5, rng.integers(-1, 2, size=E).astype(np.float32), k, "sigmoid")
    # zero tokens: nothing launched
    idx, w = moe.moe_route(torch.empty((0, 8), device="cuda"), None, 2)
    assert idx.shape == (0, 2)


def _lane_experts(E, lane):
    """Experts that segment lane `lane` of a 16-lane route segment holds (E > 64): groups of 4
    consecutive experts per lane when E is a multiple of 4 (16-byte loads), else every 16th."""
    if E % 4 == 0:
        return [e for e in range(E) if (e // 4) % 16 == lane]
    return [e for e in range(E) if e % 16 == lane]


@pytest.mark.parametrize("E,k", [(65, 8), (128, 8), (200, 6), (256, 8), (256, 9), (300, 8),
                                 (512, 8), (512, 20), (130, 64)])
def test_route_near_ties_and_crowded_lanes(E, k):
    """Selections that rest on the last bits of the logits or crowd one lane of the route's
    segment: top logits 1-3 ulp apart, one lane holding all of the largest values, +0 and -0 as
    the largest values; with and without a bias, softmax and sigmoid. Indices bit-exact."""
    rng = np.random.default_rng(E * 100 + k)
    n = 64
    l = rng.standard_normal((4 * n, E)).astype(np.float32)
    for t in range(n):                          # near ties among the top k + 1
        row = l[t]
        order = np.argsort(-row, kind="stable")
        top = row[order[0]]
        for j in range(1, min(k + 2, E)):
            row[order[j]] = np.nextafter(row[order[j - 1]], np.float32(-np.inf)) \
                if rng.random() < 0.5 else row[order[j]]
            if rng.random() < 0.2:
                row[order[j]] = np.float32(top) - np.float32(2 ** -20) * rng.integers(1, 4)
    for t in range(n, 2 * n):                   # one lane holds the largest values
        lane = int(rng.integers(0, 16))
        ex = _lane_experts(E, lane)
        l[t, ex] = 10.0 + rng.permutation(len(ex)).astype(np.float32)
    for t in range(2 * n, 3 * n):               # +0 and -0 on top of negative logits
        l[t] = -np.abs(l[t]) - 1.0
        z = rng.choice(E, size=min(E, k + 2), replace=False)
        l[t, z] = np.where(rng.random(len(z)) < 0.5, np.float32(0.0), np.float32(-0.0))
    bias = (rng.standard_normal(E) * 0.5).astype(np.float32)
    for b in (None, bias):
        for gate in ("softmax", "sigmoid"):
            _route_check(l, b, k, gate)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_layout_and_permute_full_workloads(cfg):
    w = WL.WORKLOADS[cfg]
    idx = O.route(WL.gen_logits(w), WL.gen_bias(w), w.k, w.gate)[0]
    pi = O.contiguous_placement(w.E, w.W)
    x = WL.gen_x(w)
    _layout_check(idx, pi, w.W, H=w.H, x=x, dedup=w.dedup, dst_rank=w.dst_rank)
    _layout_check(idx, None, w.W, H=w.H, x=x, dedup=not w.dedup, dst_rank=w.dst_rank, E=w.E)


def test_layout_correlated_placement_workload5():
    w = WL.WORKLOADS[5]
    idx = O.route(WL.gen_logits(w), None, w.k, w.gate)[0]
    # co-selection counts on the GPU vs the oracle
    cnt = moe.moe_coselect_counts(torch.from_numpy(idx).cuda(), w.E)
    torch.cuda.synchronize()
    Wc = O.coselect_counts(idx, w.E)
    assert np.array_equal(cnt.cpu().numpy(), Wc)
    group, _ = O.partition(Wc, w.W)
    lib_group, _ = moe.moe_placement_partition(cnt.cpu().numpy(), w.W)
    assert np.array_equal(lib_group, group)
    x = WL.gen_x(w)
    _, contig = _layout_check(idx, O.contiguous_placement(w.E, w.W), w.W, H=w.H, x=x, dedup=True)
    _, corr = _layout_check(idx, lib_group, w.W, H=w.H, x=x, dedup=True)
    # every hot pair lands on one rank, so the dedup dispatcher merges far more rows
    assert corr["D"] < contig["D"]


@pytest.mark.parametrize("N,E,k,W", [(64, 8, 2, 4), (300 * 4, 16, 3, 4), (257 * 8, 64, 8, 8),
                                     (4, 4, 4, 4), (512, 8, 1, 1), (2048, 512, 8, 64),
                                     (1024, 64, 64, 32), (40, 10, 3, 5),
                                     (40960, 256, 4, 8)])   # 160 blocks
def test_layout_edge_shapes(N, E, k, W):
    rng = np.random.default_rng(N + E + k + W)
    idx = np.argsort(rng.random((N, E)), axis=1)[:, :k].astype(np.int32)
    x = torch.from_numpy(rng.standard_normal((N, 16)).astype(np.float32))
    pi = O.contiguous_placement(E, W)[rng.permutation(E)]
    for dedup in (False, True):
        _layout_check(idx, pi, W, H=16, x=x, dedup=dedup)
        _layout_check(idx, pi, W, H=16, x=x, dedup=dedup, dst_rank=W - 1)


def test_layout_all_tokens_one_expert_and_empty_ranks():
    N, E, k, W = 1000, 16, 2, 8
    idx = np.tile(np.array([[7, 6]], np.int32), (N, 1))
    x = torch.randn(N, 8, dtype=torch.bfloat16)
    for dedup in (False, True):
        _layout_check(idx, O.contiguous_placement(E, W), W, H=8, x=x, dedup=dedup)
        _layout_check(idx, O.contiguous_placement(E, W), W, H=8, x=x, dedup=dedup, dst_rank=0)


def test_layout_deterministic():
    w = WL.WORKLOADS[3]
    idx = O.route(WL.gen_logits(w), WL.gen_bias(w), w.k, w.gate)[0]
    a, ref = _layout_check(idx, None, w.W, E=w.E)
    b, _ = _layout_check(idx, None, w.W, E=w.E)
    for f in INT_FIELDS:
        assert torch.equal(a[f], b[f]), f
    assert torch.equal(a["pair_token"][:ref["D"]], b["pair_token"][:ref["D"]])


# ---------------------------------------------------------------------------------------------
# Count rows written by the route (moe_route given the layout workspace), consumed by the layout
# with counts_ready: every layout array and permuted row equals the oracle's, and the workspace
# (the scanned count rows) equals what the layout's own count step leaves.
# ---------------------------------------------------------------------------------------------
def _counted_check(logits, bias, k, gate, placement, W, H=8, x=None, dedup=False, dst_rank=-1):
    N, E = logits.shape
    dev = torch.device("cuda")
    lg = torch.from_numpy(np.ascontiguousarray(logits, np.float32)).to(dev)
    b = None if bias is None else torch.from_numpy(np.asarray(bias, np.float32)).to(dev)
    pl = None if placement is None else torch.from_numpy(np.asarray(placement, np.int32)).to(dev)
    pi = placement if placement is not None else O.contiguous_placement(E, W)
    ridx = O.route(logits, bias, k, gate)[0]
    ref = O.layout(ridx, pi, W)
    outs = []
    for counted in (True, False):
        lay = moe.Layout(N, E, k, W, H)
        lay.ws.fill_(0xA5)                      # stale contents must not matter
        idx, _ = moe.moe_route(lg, b, k, gate, counts=(lay, pl) if counted else None)
        rows = None
        if x is not None:
            cap = (N * min(k, W) if dedup else N * k) if dst_rank < 0 else \
                (N if dedup else N * min(k, E // W))
            rows = torch.full((cap, H), float("nan"), dtype=x.dtype, device=dev)
        moe.moe_dispatch_layout(lay, idx, pl, None if x is None else x.to(dev), dedup=dedup,
                                dst_rank=dst_rank, rows_out=rows, counts_ready=counted)
        torch.cuda.synchronize()
        assert np.array_equal(idx.cpu().numpy(), ridx)
        for f in INT_FIELDS:
            assert np.array_equal(lay[f].cpu().numpy(), ref[f].reshape(-1)), (counted, f)
        D = ref["D"]
        assert np.array_equal(lay["pair_token"].cpu().numpy()[:D], ref["pair_token"])
        outs.append((lay.ws.clone(), rows))
    (ws_a, rows_a), (ws_b, rows_b) = outs
    assert torch.equal(ws_a, ws_b)
    if x is not None:
        bits = torch.int16 if x.dtype == torch.bfloat16 else torch.int32
        assert torch.equal(rows_a.view(bits), rows_b.view(bits))   # unwritten rows: same NaN
        want = O.dispatch_rows(x.float().numpy() if x.dtype == torch.bfloat16 else x.numpy(),
                               ref, dedup, dst_rank)
        wantt = torch.from_numpy(np.ascontiguousarray(want)).to(x.dtype)
        assert torch.equal(rows_a[:want.shape[0]].cpu().view(bits), wantt.view(bits))


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_route_count_rows_full_workloads(cfg):
    w = WL.WORKLOADS[cfg]
    _counted_check(WL.gen_logits(w), WL.gen_bias(w), w.k, w.gate,
                   O.contiguous_placement(w.E, w.W), w.W, H=w.H, x=WL.gen_x(w), dedup=w.dedup,
                   dst_rank=w.dst_rank)


@pytest.mark.parametrize("N,E,k,W", [(60, 1, 1, 1), (130, 2, 2, 2), (52, 3, 2, 1),
                                     (300, 4, 2, 4), (264, 8, 3, 8), (40, 10, 3, 5),
                                     (1000, 16, 2, 8), (257 * 8, 64, 8, 8), (4, 4, 4, 4),
                                     (2048, 512, 8, 64), (1024, 64, 64, 32),
                                     (4104, 256, 8, 8)])
def test_route_count_rows_edge_shapes(N, E, k, W):
    # every lane width of the route (1, 2, 4, 8, 16 lanes per token: count rows of 64, 64, 64,
    # 32 and 16 tokens), token counts that end inside a row and inside a 256-token block, integer
    # logits with heavy ties, permuted placements, W = 1 and W = 64, k = E
    rng = np.random.default_rng(N * 7 + E + k + W)
    logits = rng.integers(-3, 4, size=(N, E)).astype(np.float32)
    pi = O.contiguous_placement(E, W)[rng.permutation(E)]
    x = torch.from_numpy(rng.standard_normal((N, 16)).astype(np.float32))
    for dedup in (False, True):
        _counted_check(logits, None, k, "softmax", pi, W, H=16, x=x, dedup=dedup)
        _counted_check(logits, None, k, "softmax", None, W, H=16, x=x, dedup=dedup,
                       dst_rank=W - 1)
