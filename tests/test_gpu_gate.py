"""GPU parity of the router linear layer + route (moe_gate_route) against the CPU oracle.

Logits: within 1e-5 of max|logit| (the gate keeps fp32 weights: a bf16 high part plus a bf16
remainder, fp32 accumulation; the oracle sums in fp64). Selection: bit-exact against the
oracle's route run on the GPU's own logits (the decision taken in the kernel's precision);
weights within 1e-4 relative."""
import numpy as np
import pytest
import torch

from dispatch_expert_gemm_amd import moe
from dispatch_expert_gemm_amd import workloads as WL
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu

LOGIT_TOL = 1e-5


def _check(x, w_router, bias, k, gate, tol=LOGIT_TOL):
    dev = torch.device("cuda")
    xd = x.to(dev)
    wd = torch.from_numpy(np.ascontiguousarray(w_router, np.float32)).to(dev)
    bd = None if bias is None else torch.from_numpy(np.asarray(bias, np.float32)).to(dev)
    logits, idx, w = moe.moe_gate_route(xd, wd, bd, k, gate)
    torch.cuda.synchronize()
    ref = O.gate_logits(x.float().numpy(), w_router).astype(np.float64)
    got = logits.cpu().numpy()
    err = np.abs(got.astype(np.float64) - ref).max() / max(np.abs(ref).max(), 1e-30)
    assert err <= tol, err
    ridx, rw = O.route(got, bias, k, gate)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    rel = np.abs(w.cpu().numpy().astype(np.float64) - rw) / np.abs(rw)
    assert rel.max() <= 1e-4
    return got


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_gate_route_shrunk_workloads(cfg):
    """The workloads' distributions and E, k, gate and bias at 1000 tokens of width 512
    (1000 is not a multiple of the 64-token tile)."""
    w = WL.WORKLOADS[cfg]
    w = WL.shrink(w, N=min(w.N, 1000), H=min(w.H, 512))
    _check(WL.gen_x(w), WL.gen_router(w), WL.gen_bias(w), w.k, w.gate)


@pytest.mark.parametrize("N,H,E,k,dt", [(1, 32, 1, 1, "bf16"), (63, 64, 5, 2, "f32"),
                                         (65, 96, 33, 3, "bf16"), (130, 160, 100, 7, "f32"),
                                         (200, 256, 256, 8, "bf16"), (64, 2048, 128, 6, "bf16"),
                                         (257, 128, 64, 64, "f32"),
                                         # route fused into the gate epilogue: 64 x 64 tiles
                                         # (33-64 experts, 16384 tokens or more) and 32 x 32
                                         (16400, 64, 48, 5, "bf16"), (100, 64, 20, 3, "f32"),
                                         # 128 x 128 tiles: a partial last token tile and a
                                         # partial second expert tile
                                         (16421, 512, 200, 8, "bf16"),
                                         (16421, 256, 129, 4, "f32"),
                                         # 5-32 experts: 32-token tiles, K steps of 64 (fewer
                                         # steps than the ring holds, 16 or 32 router rows
                                         # copied, bf16 and fp32 x, ragged last tile)
                                         (300, 192, 24, 3, "bf16"), (33, 64, 32, 4, "bf16"),
                                         (777, 320, 9, 2, "f32"), (2000, 1024, 17, 5, "f32"),
                                         # the 64-token tiles again: 4 experts (64-token count
                                         # rows), H not a multiple of 64, 17-32 experts on more
                                         # than 16384 tokens
                                         (500, 128, 4, 2, "bf16"), (200, 96, 12, 2, "bf16"),
                                         (16420, 64, 24, 2, "bf16")])
def test_gate_route_ragged_shapes(N, H, E, k, dt):
    rng = np.random.default_rng(N * 7 + E)
    x = torch.from_numpy(rng.standard_normal((N, H)).astype(np.float32))
    if dt == "bf16":
        x = x.to(torch.bfloat16)
    wr = (rng.standard_normal((E, H)) * 0.05).astype(np.float32)
    _check(x, wr, None, k, "softmax")


def test_gate_identity_router_is_exact():
    # W_R picks coordinates: bf16 x passes through the split product exactly
    rng = np.random.default_rng(9)
    x = torch.from_numpy(rng.standard_normal((96, 64)).astype(np.float32)).to(torch.bfloat16)
    wr = np.zeros((40, 64), np.float32)
    wr[np.arange(40), rng.permutation(64)[:40]] = 1.0
    got = _check(x, wr, None, 4, "softmax", tol=0.0)
    assert np.array_equal(got, O.gate_logits(x.float().numpy(), wr))


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_gate_route_full_workloads_every_token(cfg):
    """Full-size shapes through the same launch the benchmark's fused-gate mode uses; every
    token's logits against the fp64 oracle, every token's selection against the oracle's route
    on the GPU's logits."""
    w = WL.WORKLOADS[cfg]
    dev = torch.device("cuda")
    x = WL.gen_x(w)
    wr = WL.gen_router(w)
    bias = WL.gen_bias(w)
    logits, idx, wt = moe.moe_gate_route(
        x.to(dev), torch.from_numpy(wr).to(dev),
        None if bias is None else torch.from_numpy(bias).to(dev), w.k, w.gate)
    torch.cuda.synchronize()
    ref = O.gate_logits(x.float().numpy(), wr).astype(np.float64)
    got = logits.cpu().numpy()
    err = np.abs(got.astype(np.float64) - ref).max() / np.abs(ref).max()
    assert err <= LOGIT_TOL, err
    ridx, rw = O.route(got, bias, w.k, w.gate)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert (np.abs(wt.cpu().numpy().astype(np.float64) - rw) / np.abs(rw)).max() <= 1e-4
    print(f"[gate {w.name}] {w.N} tokens: logits within {err:.2e} of max, selection bit-exact",
          flush=True)


@pytest.mark.parametrize("N,H,E,k,W,dt", [(1000, 64, 16, 1, 4, "bf16"),    # 32-token tiles,
                                           (328, 64, 8, 2, 8, "f32"),        # 16 and 8 lanes
                                           (1000, 192, 24, 3, 4, "bf16"),    # 32 router rows
                                           (776, 128, 32, 4, 8, "f32"),
                                           (96, 64, 4, 2, 2, "bf16"),        # fused, 4 lanes
                                           (130, 64, 2, 1, 1, "f32"),        # fused, 2 lanes
                                           (1000, 128, 64, 6, 8, "bf16"),    # unfused 64 x 32
                                           (16400, 64, 48, 5, 8, "bf16"),    # fused 64 x 64
                                           (520, 64, 128, 8, 8, "bf16"),     # fused 64 x 128
                                           (2056, 64, 256, 8, 8, "f32"),     # fused 64 x 256
                                           (16392, 64, 256, 8, 8, "bf16")])  # 128 x 128, unfused
def test_gate_count_rows_feed_the_layout(N, H, E, k, W, dt):
    """moe_gate_route given the layout workspace writes the count rows (in its fused epilogue,
    or through the route kernel where the product is not fused); the layout then skips its count
    step and every array equals the oracle's layout of the GPU's own selection, and the scanned
    workspace equals the one the layout's own count step leaves."""
    rng = np.random.default_rng(N + E)
    dev = torch.device("cuda")
    x = torch.from_numpy(rng.standard_normal((N, H)).astype(np.float32))
    if dt == "bf16":
        x = x.to(torch.bfloat16)
    wr = torch.from_numpy((rng.standard_normal((E, H)) * 0.05).astype(np.float32)).to(dev)
    pi = O.contiguous_placement(E, W)[rng.permutation(E)]
    pl = torch.from_numpy(pi.astype(np.int32)).to(dev)
    xd = x.to(dev)
    lay = moe.Layout(N, E, k, W, 8)
    lay.ws.fill_(0x5A)
    _, idx, _ = moe.moe_gate_route(xd, wr, None, k, "softmax", counts=(lay, pl))
    moe.moe_dispatch_layout(lay, idx, pl, counts_ready=True)
    ref_lay = moe.Layout(N, E, k, W, 8)
    ref_lay.ws.fill_(0x5A)                      # the same bytes in the alignment padding
    moe.moe_dispatch_layout(ref_lay, idx, pl)
    torch.cuda.synchronize()
    ref = O.layout(idx.cpu().numpy(), pi, W)
    for f in ("expert_counts", "expert_offsets", "group_offsets", "rank_counts", "rank_offsets",
              "send_counts", "row_of_slot", "slot_of_row", "pair_counts", "pair_offsets",
              "pair_of_slot", "pair_send_counts", "expand_src"):
        assert np.array_equal(lay[f].cpu().numpy(), ref[f].reshape(-1)), f
    assert torch.equal(lay.ws, ref_lay.ws)


@pytest.mark.parametrize("N,H,E,k,dt", [(1000, 512, 16, 1, "bf16"), (1000, 256, 64, 6, "bf16"),
                                         (2056, 128, 256, 8, "f32"), (16392, 64, 256, 8, "bf16")])
def test_gate_prepared_split_is_identical(N, H, E, k, dt):
    """The router weights split once (moe_gate_prepare, then w_router NULL) give the same
    logits and selection bits as the split on every call."""
    rng = np.random.default_rng(N + H)
    dev = torch.device("cuda")
    x = torch.from_numpy(rng.standard_normal((N, H)).astype(np.float32))
    if dt == "bf16":
        x = x.to(torch.bfloat16)
    xd = x.to(dev)
    wr = torch.from_numpy((rng.standard_normal((E, H)) * 0.05).astype(np.float32)).to(dev)
    l1, i1, w1 = moe.moe_gate_route(xd, wr, None, k)
    ws = moe.moe_gate_prepare(wr)
    l2, i2, w2 = moe.moe_gate_route(xd, wr, None, k, workspace=ws, prepared=True)
    l3, i3, w3 = moe.moe_gate_route(xd, wr, None, k, workspace=ws, prepared=True)   # reused
    torch.cuda.synchronize()
    for a, b in ((l1, l2), (i1, i2), (w1, w2), (l2, l3), (i2, i3), (w2, w3)):
        assert torch.equal(a, b)


def test_gate_binding_checks_shapes():
    dev = torch.device("cuda")
    x = torch.zeros((64, 256), dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError):
        moe.moe_gate_route(x, torch.zeros((8, 128), device=dev), None, 2)      # H mismatch
    with pytest.raises(ValueError):
        moe.moe_gate_route(x, torch.zeros((8, 256), device=dev), None, 2,
                           workspace=torch.empty(16, dtype=torch.uint8, device=dev))
    with pytest.raises(ValueError):
        moe.moe_gate_route(x, torch.zeros((8, 256), device=dev), None, 2,
                           logits=torch.empty((64, 7), device=dev))
