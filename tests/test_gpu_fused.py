"""GPU parity of the one-launch layer for small batches (moe_layer_fused) against the CPU oracle:
the routing bit-exact, every token of the output within the dtype's tolerance and the
element-wise error bound; repeated launches and graph replays bit-identical (the launch returns
its device-wide counters to zero); the stage waits never give up."""
import numpy as np
import pytest
import torch

from dispatch_expert_gemm_amd import moe
from dispatch_expert_gemm_amd import workloads as WL
from dispatch_expert_gemm_amd.layer import FusedLayerRun, MoELayerRun
from oracle import moe_oracle as O
from tests import parity as P

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def _check_fused(w, repeats=2, pack=None):
    print(f"[fused {w.name} N={w.N} pack={pack}] start", flush=True)
    run = MoELayerRun(w, pack=pack)
    f = FusedLayerRun(run)
    f.step()
    assert f.error() == 0, "a stage wait gave up"
    idx, wts = O.route(WL.gen_logits(w), WL.gen_bias(w), w.k, w.gate)
    assert np.array_equal(f.topk_idx.cpu().numpy(), idx)
    assert (np.abs(f.topk_w.cpu().numpy().astype(np.float64) - wts) / np.abs(wts)).max() <= 1e-4
    wgu, wd = run.host["experts"]
    experts = {e: (wgu[i], wd[i]) for i, e in enumerate(run.local)}
    shared = [WL.gen_shared(w, s) for s in range(w.n_shared)]
    tokens = np.arange(w.N)
    ref, bnd = P.expected_out(w, WL.gen_x(w), idx, wts, experts, shared, tokens, with_bound=True)
    got = f.out.cpu()
    err, ratio = P.rel_err(got, ref), P.elem_ratio(got, ref, bnd)
    print(f"[fused {w.name} N={w.N}] max relative error {err:.3e}, element-wise {ratio:.3f} of "
          f"the bound", flush=True)
    assert err <= P.TOL[w.dtype] and ratio <= 1.0
    first = f.out.clone()
    for _ in range(repeats):
        f.out.fill_(float("nan"))
        f.step()
        assert f.error() == 0
        assert torch.equal(_bits(first), _bits(f.out))
    return f


def test_fused_tiny_fp32():
    _check_fused(WL.WORKLOADS[1])


@pytest.mark.parametrize("pack", [True, False])
@pytest.mark.parametrize("N", [64, 256, 512])
def test_fused_dsv2_lite_small_batches(N, pack):
    # the DeepSeek-V2-Lite-shaped layer (H 2048, 64 experts top-6, I 1408, 2 shared experts,
    # bias) at decode batch sizes, on packed and on plain weights
    _check_fused(WL.shrink(WL.WORKLOADS[2], N=N), pack=pack)


@pytest.mark.parametrize("N,E,k,H,I,S,dt", [(100, 8, 2, 128, 256, 1, "f32"),
                                             (520, 4, 1, 256, 384, 0, "bf16"),
                                             (40, 512, 8, 128, 128, 0, "bf16"),
                                             (1000, 16, 4, 128, 128, 2, "bf16"),
                                             (1024, 64, 4, 256, 128, 1, "bf16")])
def test_fused_edge_shapes(N, E, k, H, I, S, dt):
    # N not a multiple of anything; groups of more than 128 rows (several row chunks; E = 4
    # gives every expert ~130 rows); 512 experts with most groups empty; N * k = 4000; the
    # limits themselves: N = 1024 tokens and N * k = 4096 slots
    base = WL.WORKLOADS[2 if dt == "bf16" else 1]
    W = 4 if E % 4 == 0 and N % 4 == 0 else 1
    w = WL.shrink(base, N=N, E=E, k=k, H=H, I=I, W=W).replace(n_shared=S, dedup=False)
    _check_fused(w, repeats=1)


def test_fused_graph_replays():
    w = WL.shrink(WL.WORKLOADS[2], N=128)
    run = MoELayerRun(w)
    f = FusedLayerRun(run)
    f.step()
    torch.cuda.synchronize()
    eager = f.out.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        f.step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        f.step()
    for _ in range(3):
        f.out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert f.error() == 0
        assert torch.equal(_bits(eager), _bits(f.out))


def test_fused_matches_multi_launch_routing():
    # the same routing and layout decisions as the library's separate launches
    w = WL.shrink(WL.WORKLOADS[2], N=256)
    run = MoELayerRun(w)
    f = FusedLayerRun(run)
    f.step()
    run.step()
    torch.cuda.synchronize()
    assert torch.equal(f.topk_idx, run.topk_idx)
    assert torch.equal(f.topk_w, run.topk_w)
    assert P.rel_err(f.out.cpu(), P.f64(run.out.cpu())) <= 1e-2


def test_fused_binding_checks():
    dev = torch.device("cuda")
    x = torch.zeros((64, 128), dtype=torch.bfloat16, device=dev)
    lg = torch.zeros((64, 8), device=dev)
    wgu = torch.zeros((8, 256, 128), dtype=torch.bfloat16, device=dev)
    wd = torch.zeros((8, 128, 128), dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError):
        moe.moe_layer_fused(x, lg, None, 2, "softmax", wgu, wd[:, :64])     # H mismatch
    with pytest.raises(ValueError):
        moe.moe_layer_fused(x, lg[:, :4], None, 2, "softmax", wgu, wd)      # E mismatch
