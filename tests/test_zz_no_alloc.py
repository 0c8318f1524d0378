"""The dispatch layout entry point that allocates nothing (its workspace is the library's fixed
device array) against moe_dispatch_layout with a caller workspace: identical layout arrays and
dispatched rows, bit for bit, on two calls in a row, the second on a smaller problem (the array
keeps the first call's contents)."""
import numpy as np
import pytest
import torch

from dispatch_expert_gemm_amd import moe

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda")


def _problem(seed, N, E, k, H, dtype):
    rng = np.random.default_rng(seed)
    idx = np.argsort(rng.random((N, E)), axis=1)[:, :k].astype(np.int32)
    x = torch.from_numpy(rng.standard_normal((N, H)).astype(np.float32)).to(dtype)
    return torch.from_numpy(idx).to(DEV), x.to(DEV)


def _rows_cap(N, E, k, W, dedup, dst_rank):
    if dst_rank < 0:
        return N * min(k, W) if dedup else N * k
    return N if dedup else N * min(k, E // W)


@pytest.mark.parametrize("order", ["large-then-small"])
def test_noalloc_matches_workspace_call(order):
    cases = [dict(seed=1, N=16384, E=256, k=8, W=8, H=512, dtype=torch.bfloat16, dedup=True,
                  dst_rank=0),
             dict(seed=2, N=512, E=16, k=6, W=8, H=256, dtype=torch.float32, dedup=False,
                  dst_rank=-1)]
    for c in cases:
        print(f"[noalloc] N={c['N']} E={c['E']} k={c['k']} W={c['W']} dedup={c['dedup']} "
              f"dst_rank={c['dst_rank']}", flush=True)
        idx, x = _problem(c["seed"], c["N"], c["E"], c["k"], c["H"], c["dtype"])
        cap = _rows_cap(c["N"], c["E"], c["k"], c["W"], c["dedup"], c["dst_rank"])
        outs = []
        for fn in (moe.moe_dispatch_layout, moe.moe_dispatch_layout_noalloc):
            lay = moe.Layout(c["N"], c["E"], c["k"], c["W"], c["H"], device=DEV)
            lay.buf.fill_(-7)
            rows = torch.full((cap, c["H"]), float("nan"), dtype=c["dtype"], device=DEV)
            fn(lay, idx, None, x, dedup=c["dedup"], dst_rank=c["dst_rank"], rows_out=rows)
            torch.cuda.synchronize()
            outs.append((lay, rows))
        (la, ra), (lb, rb) = outs
        for f in moe.LAYOUT_FIELDS:
            assert torch.equal(la[f], lb[f]), f
        assert torch.equal(ra.view(torch.int16) if ra.dtype == torch.bfloat16 else ra.view(torch.int32),
                           rb.view(torch.int16) if rb.dtype == torch.bfloat16 else rb.view(torch.int32))
