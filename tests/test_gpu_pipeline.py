"""GPU checks of the microbatch-pipelined layer step (blog "Kernel fusion for expert
parallelism", section "Fusing the layer into one kernel": microbatches pipelined through the
layer's stages): every token's output bit-identical to the unsplit step, whose own parity against
the oracle is checked below as well."""
import numpy as np
import pytest
import torch

from dispatch_expert_gemm_amd import workloads as WL
from dispatch_expert_gemm_amd.layer import MicrobatchLayer
from oracle import moe_oracle as O
from tests import parity as P

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg,kw,M", [(1, {}, 2), (1, {}, 4),
                                      (2, dict(N=1024, H=256, E=16, k=6, W=8, I=256), 2),
                                      (2, dict(N=1024, H=256, E=16, k=6, W=8, I=256), 4),
                                      (4, dict(N=512, H=256, E=16, k=1, W=4, I=384), 4),
                                      (5, dict(N=2048), 2), (2, {}, 2)])
def test_microbatch_step_matches_whole_step(cfg, kw, M):
    w = WL.shrink(WL.WORKLOADS[cfg], **kw) if kw else WL.WORKLOADS[cfg]
    mb = MicrobatchLayer(w, M)
    mb.full.step()
    torch.cuda.synchronize()
    want = mb.full.out.clone()
    for _ in range(2):                       # the second pass reuses every buffer
        for r in mb.subs:
            r.out.zero_()
        mb.step()
        torch.cuda.synchronize()
        got = mb.outputs()
        if want.dtype == torch.bfloat16:
            assert torch.equal(got.view(torch.int16), want.view(torch.int16))
        else:
            assert torch.equal(got, want)
    # the whole step against the oracle on a few tokens
    f = mb.full
    x = P.f64(f.host["x"])
    if w.expert != "identity":   # the host copies (the device ones may be in the packed layout)
        wgu, wd = f.host["experts"]
        sgu, sd = f.host["shared"]
    idx, wts = O.route(np.asarray(f.host["logits"]), f.host["bias"], w.k, w.gate)
    toks = np.arange(0, w.N, max(1, w.N // 16))
    ref = np.zeros((len(toks), w.H))
    for n, t in enumerate(toks):
        for j in range(w.k):
            e = idx[t, j]
            if w.expert == "identity":
                ye = x[t]
            else:
                ye = O.swiglu_expert(x[t:t + 1], P.f64(wgu[e]), P.f64(wd[e]))[0]
            ref[n] += wts[t, j] * ye
        for s in range(w.n_shared):
            ref[n] += O.swiglu_expert(x[t:t + 1], P.f64(sgu[s]), P.f64(sd[s]))[0]
    key = "f32" if want.dtype == torch.float32 else "bf16"
    assert P.rel_err(want[toks].cpu(), ref) <= P.TOL[key]


def test_microbatch_rejects_uneven_splits():
    w = WL.shrink(WL.WORKLOADS[2], N=1024, H=256, E=16, k=6, W=8, I=256)
    with pytest.raises(ValueError):
        MicrobatchLayer(w, 3)
    with pytest.raises(ValueError):
        MicrobatchLayer(WL.shrink(WL.WORKLOADS[3], N=2048, H=256, E=32, I=256), 2)


def test_device_info_matches_runtime():
    from dispatch_expert_gemm_amd import moe
    cus, lds, clk, mclk = moe.moe_device_info()
    props = torch.cuda.get_device_properties(0)
    assert cus == props.multi_processor_count
    assert lds >= 64 * 1024 and clk > 0 and mclk > 0
