"""GPU parity of the grouped SwiGLU FFN at the largest operand blocks its 32-bit byte offsets
allow: rows x H x 2 bytes just below 4 GiB (the host rejects one row more), routed groups and a
shared expert, checked against the CPU oracle on sampled rows that include the last ones."""
import numpy as np
import pytest
import torch

from dispatch_expert_gemm_amd import moe
from oracle import moe_oracle as O
from tests import parity as P

pytestmark = pytest.mark.gpu

H, I = 7168, 256
ROWS = (2 ** 32 - 1) // (2 * H) - 1      # the most rows the host accepts at this H


@pytest.mark.timeout(600)
def test_ffn_operand_blocks_just_below_4_gib():
    assert (ROWS + 1) * H * 2 <= 2 ** 32 - 1 < (ROWS + 2) * H * 2
    g = torch.Generator(device="cuda").manual_seed(4242)
    sizes = [ROWS // 2 + 1, ROWS - ROWS // 2 - 1]
    offs = torch.tensor(np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32), device="cuda")
    a = torch.randn((ROWS, H), device="cuda", dtype=torch.bfloat16, generator=g)
    w_gu = torch.randn((2, 2 * I, H), device="cuda", dtype=torch.bfloat16, generator=g) * H ** -0.5
    w_d = torch.randn((2, H, I), device="cuda", dtype=torch.bfloat16, generator=g) * I ** -0.5
    s_gu = torch.randn((1, 2 * I, H), device="cuda", dtype=torch.bfloat16, generator=g) * H ** -0.5
    s_d = torch.randn((1, H, I), device="cuda", dtype=torch.bfloat16, generator=g) * I ** -0.5
    h = torch.empty((ROWS, I), device="cuda", dtype=torch.bfloat16)
    y = torch.empty((ROWS, H), device="cuda", dtype=torch.bfloat16)
    sh_h = torch.empty((1, ROWS, I), device="cuda", dtype=torch.bfloat16)
    sh_y = torch.empty((1, ROWS, H), device="cuda", dtype=torch.bfloat16)
    # routed groups over all rows, and one shared expert whose block is the same ROWS rows
    moe.moe_expert_ffn(a, offs, 2, w_gu, w_d, h, y, ROWS, shared_x=a, shared_w_gate_up=s_gu,
                       shared_w_down=s_d, shared_h=sh_h, shared_y=sh_y)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([[0, sizes[0] - 1, sizes[0], ROWS - 2, ROWS - 1],
                                     np.arange(ROWS - 40, ROWS),
                                     rng.integers(0, ROWS, 24)]))
    x = P.f64(a[torch.from_numpy(rows).cuda()])
    grp = (rows >= sizes[0]).astype(np.int64)
    ref = np.stack([O.swiglu_expert(x[i:i + 1], P.f64(w_gu[grp[i]]), P.f64(w_d[grp[i]]))[0]
                    for i in range(len(rows))])
    assert P.rel_err(y[torch.from_numpy(rows).cuda()].cpu(), ref) <= P.TOL["bf16"]
    ref_sh = O.swiglu_expert(x, P.f64(s_gu[0]), P.f64(s_d[0]))
    assert P.rel_err(sh_y[0][torch.from_numpy(rows).cuda()].cpu(), ref_sh) <= P.TOL["bf16"]
