"""A whole layer step recorded into a HIP graph and replayed: every replay, with eager work and
synchronisations between replays and the inputs changed in place before some of them, must give
bit-identical outputs to an eager step on the same inputs (the kernels are deterministic)."""
import numpy as np
import pytest
import torch

from dispatch_expert_gemm_amd import workloads as WL
from dispatch_expert_gemm_amd.layer import MoELayerRun

pytestmark = pytest.mark.gpu


def _outputs(run):
    return [run.out.clone(), run.topk_idx.clone(), run.topk_w.clone()]


@pytest.mark.parametrize("cfg,kw", [(1, {}), (2, dict(N=512, H=256, E=16, k=6, W=8, I=256)),
                                    (5, dict(N=2048)), (4, dict(N=512, H=256, E=16, k=1, W=4,
                                                                 I=384))])
def test_graph_replays_match_eager(cfg, kw):
    w = WL.shrink(WL.WORKLOADS[cfg], **kw) if kw else WL.WORKLOADS[cfg]
    run = MoELayerRun(w)
    run.step()
    run.place_standins()
    torch.cuda.synchronize()
    g = run.capture()
    rng = np.random.default_rng(cfg)
    for rep in range(4):
        if rep >= 2:   # new inputs in place
            run.logits.copy_(torch.from_numpy(
                rng.standard_normal(tuple(run.logits.shape)).astype(np.float32)))
            run.x.copy_(torch.from_numpy(
                rng.standard_normal(tuple(run.x.shape)).astype(np.float32)).to(run.x.dtype))
        g.replay()
        torch.cuda.synchronize()
        got = _outputs(run)
        _ = torch.ones(1 << 20, device="cuda").sum().item()   # unrelated eager work
        run.step()
        torch.cuda.synchronize()
        want = _outputs(run)
        for a, b in zip(got, want):
            assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else
                               a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int32) if b.dtype == torch.float32 else
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b), rep


@pytest.mark.parametrize("cfg,kw", [
    # 32-token tiles (5-32 experts), the route in the epilogue
    (2, dict(N=512, H=256, E=16, k=6, W=8, I=256)),
    # 128 x 128 tiles on eight waves (two K groups), then the route kernel
    (2, dict(N=16384, H=256, E=256, k=8, W=8, I=256)),
    # fp32 x, 64 x 64 tiles on eight waves with the route in the epilogue
    (5, dict(N=16384, H=256, E=64, k=2, W=32))])
def test_graph_with_fused_gate(cfg, kw):
    w = WL.shrink(WL.WORKLOADS[cfg], **kw)
    run = MoELayerRun(w)
    run.step(fused_gate=True)
    torch.cuda.synchronize()
    g = run.capture(fused_gate=True)
    for _ in range(3):
        g.replay()
        torch.cuda.synchronize()
        got = _outputs(run)
        run.step(fused_gate=True)
        torch.cuda.synchronize()
        for a, b in zip(got, _outputs(run)):
            assert torch.equal(a, b)


@pytest.mark.parametrize("cfg,kw", [(2, dict(N=512, H=256, E=16, k=6, W=8, I=256)),
                                    (4, dict(N=512, H=256, E=16, k=1, W=4, I=384))])
def test_overlapped_shared_experts(cfg, kw):
    # shared experts on a second stream while route and dispatch run: bit-identical to the
    # single-stream step, eagerly and as a captured graph (fork and join inside the capture)
    w = WL.shrink(WL.WORKLOADS[cfg], **kw)
    run = MoELayerRun(w)
    run.step()
    torch.cuda.synchronize()
    want = _outputs(run)
    run.out.zero_()
    run.step(overlap_shared=True)
    torch.cuda.synchronize()
    for a, b in zip(_outputs(run), want):
        assert torch.equal(a, b)
    g = run.capture(overlap_shared=True)
    rng = np.random.default_rng(cfg)
    for rep in range(3):
        run.x.copy_(torch.from_numpy(
            rng.standard_normal(tuple(run.x.shape)).astype(np.float32)).to(run.x.dtype))
        g.replay()
        torch.cuda.synchronize()
        got = _outputs(run)
        run.step()
        torch.cuda.synchronize()
        for a, b in zip(got, _outputs(run)):
            assert torch.equal(a, b), rep


@pytest.mark.parametrize("dedup", [False, True])
def test_graph_one_rank_share(dedup):
    # one rank's share for rank 3 (its partition starts past row 0): the step reads nothing
    # back on the host, so it records into a graph, and replays match eager steps bit for bit
    w = WL.shrink(WL.WORKLOADS[3], N=1024, H=256, E=32, k=8, W=8, I=256, dst_rank=3,
                  dedup=dedup)
    run = MoELayerRun(w)
    run.route()
    run.dispatch()
    run.place_standins()
    run.step()
    torch.cuda.synchronize()
    g = run.capture()
    rng = np.random.default_rng(33)
    for rep in range(3):
        run.x.copy_(torch.from_numpy(
            rng.standard_normal(tuple(run.x.shape)).astype(np.float32)).to(run.x.dtype))
        g.replay()
        torch.cuda.synchronize()
        got = _outputs(run)
        run.step()
        torch.cuda.synchronize()
        for a, b in zip(got, _outputs(run)):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b), rep
