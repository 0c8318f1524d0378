"""Packed expert weights: moe_pack_weights is the permutation its header defines (checked bit for
bit against a host transcription of that definition), and the grouped FFN on packed weights
matches the oracle on ragged groups, group tails, the dedup gather and shared experts."""
import numpy as np
import pytest
import torch

from dispatch_expert_gemm_amd import moe
from oracle import moe_oracle as O
from tests import parity as P

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda")


def _host_pack(w: np.ndarray, NB: int) -> np.ndarray:
    """The packed layout written out from its definition: for group g, panel p, K step kt, chunk
    q and lane l, the 8 values W[row][kt*64 + 8*c : +8] with r = 8q + l//8,
    c = (l % 8) ^ ((r // 2) % 8)."""
    G, R, K = w.shape
    Nn = R // NB
    KT = K // 64
    prow = 128 if NB == 2 else 256
    panels = Nn // prow
    out = np.empty((G, panels, KT, 32, 64, 8), dtype=w.dtype)
    q = np.arange(32)[:, None]
    l = np.arange(64)[None, :]
    r = 8 * q + l // 8
    c = (l % 8) ^ ((r // 2) % 8)
    for p in range(panels):
        if NB == 2:
            row = np.where(r < 128, 128 * p + r, Nn + 128 * p + r - 128)
        else:
            row = 256 * p + r
        for kt in range(KT):
            cols = kt * 64 + 8 * c[..., None] + np.arange(8)          # [32, 64, 8]
            out[:, p, kt] = w[:, row[..., None], cols]
    return out.reshape(G, R, K)


@pytest.mark.parametrize("NB,Nn,K", [(2, 128, 128), (2, 384, 256), (1, 256, 192), (1, 512, 64)])
def test_pack_weights_is_the_defined_permutation(NB, Nn, K):
    rng = np.random.default_rng(NB * 1000 + Nn + K)
    G = 3
    bits = rng.integers(0, 1 << 16, size=(G, NB * Nn, K), dtype=np.uint16)
    w = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    got = moe.moe_pack_weights(w, NB)
    torch.cuda.synchronize()
    want = _host_pack(bits, NB)
    assert np.array_equal(got.view(torch.int16).cpu().numpy().view(np.uint16), want)


def _rand(rng, shape, std):
    return torch.from_numpy((rng.standard_normal(shape) * std).astype(np.float32)).to(
        torch.bfloat16)


@pytest.mark.parametrize("sizes", [[0, 1, 127, 128, 300, 64, 0, 129],
                                   [1100, 0, 513, 256, 767, 1],
                                   [384, 129, 640, 0, 1024, 300, 128]],
                         ids=["small", "large", "tails"])
@pytest.mark.parametrize("H,I", [(256, 256), (512, 384)])
@pytest.mark.parametrize("gather", [False, True])
def test_ffn_on_packed_weights(sizes, H, I, gather):
    rng = np.random.default_rng(H + I + len(sizes) + gather)
    G = len(sizes)
    base = 37
    offs = np.concatenate([[0], np.cumsum(sizes)]) + base
    R = int(offs[-1] - base)
    x = _rand(rng, (R, H), 1.0)
    if gather:
        perm = rng.permutation(R)
        src = torch.empty_like(x)
        src[perm] = x
        gmap = np.full(int(offs[-1]), -1, np.int32)
        gmap[base:] = perm + 5
        rows, gmap_d = src.to(DEV), torch.from_numpy(gmap).to(DEV)
        gbase = torch.tensor([5], dtype=torch.int32, device=DEV)
    else:
        rows, gmap_d, gbase = x.to(DEV), None, None
    w_gu = _rand(rng, (G, 2 * I, H), H ** -0.5)
    w_d = _rand(rng, (G, H, I), I ** -0.5)
    S, M_sh = 1, 200
    xs = _rand(rng, (M_sh, H), 1.0)
    s_gu = _rand(rng, (S, 2 * I, H), H ** -0.5)
    s_d = _rand(rng, (S, H, I), I ** -0.5)
    offs_d = torch.from_numpy(offs.astype(np.int32)).to(DEV)
    outs = []
    for packed in (False, True):
        pk = (lambda t, nb: moe.moe_pack_weights(t.to(DEV), nb)) if packed else \
             (lambda t, nb: t.to(DEV))
        h = torch.empty((R, I), dtype=torch.bfloat16, device=DEV)
        y = torch.full((R, H), float("nan"), dtype=torch.bfloat16, device=DEV)
        sh_h = torch.empty((S, M_sh, I), dtype=torch.bfloat16, device=DEV)
        sh_y = torch.full((S, M_sh, H), float("nan"), dtype=torch.bfloat16, device=DEV)
        moe.moe_expert_ffn(rows, offs_d, G, pk(w_gu, 2), pk(w_d, 1), h, y, R, row_gather=gmap_d,
                           gather_base=gbase, shared_x=xs.to(DEV),
                           shared_w_gate_up=pk(s_gu, 2), shared_w_down=pk(s_d, 1),
                           shared_h=sh_h, shared_y=sh_y, weights_packed=packed)
        torch.cuda.synchronize()
        outs.append((y.cpu(), sh_y.cpu()))
    ref = np.zeros((R, H))
    for g in range(G):
        lo, hi = offs[g] - base, offs[g + 1] - base
        if hi > lo:
            ref[lo:hi] = O.swiglu_expert(P.f64(x[lo:hi]), P.f64(w_gu[g]), P.f64(w_d[g]))
    rs = O.swiglu_expert(P.f64(xs), P.f64(s_gu[0]), P.f64(s_d[0]))
    for y, sh_y in outs:
        assert P.rel_err(y, ref) <= P.TOL["bf16"]
        assert P.rel_err(sh_y[0], rs) <= P.TOL["bf16"]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_ffn_bit_identical_under_cu_caps(dtype):
    """moe_set_gemm_max_cus changes only the persistent grid: with 8 (several rounds of tiles
    per workgroup), 24 and 64 compute units the outputs equal the full grid's bit for bit."""
    rng = np.random.default_rng(7)
    sizes = [1100, 0, 513, 256, 767, 1]
    H, I = 512, 384
    G = len(sizes)
    offs = np.concatenate([[0], np.cumsum(sizes)])
    R = int(offs[-1])
    x = _rand(rng, (R, H), 1.0).to(dtype).to(DEV)
    w_gu = _rand(rng, (G, 2 * I, H), H ** -0.5).to(dtype).to(DEV)
    w_d = _rand(rng, (G, H, I), I ** -0.5).to(dtype).to(DEV)
    xs = _rand(rng, (300, H), 1.0).to(dtype).to(DEV)
    s_gu = _rand(rng, (1, 2 * I, H), H ** -0.5).to(dtype).to(DEV)
    s_d = _rand(rng, (1, H, I), I ** -0.5).to(dtype).to(DEV)
    offs_d = torch.from_numpy(offs.astype(np.int32)).to(DEV)
    outs = []
    try:
        for cap in (0, 8, 24, 64):
            moe.moe_set_gemm_max_cus(cap)
            h = torch.empty((R, I), dtype=dtype, device=DEV)
            y = torch.full((R, H), float("nan"), dtype=dtype, device=DEV)
            sh_h = torch.empty((1, 300, I), dtype=dtype, device=DEV)
            sh_y = torch.full((1, 300, H), float("nan"), dtype=dtype, device=DEV)
            moe.moe_expert_ffn(x, offs_d, G, w_gu, w_d, h, y, R, shared_x=xs,
                               shared_w_gate_up=s_gu, shared_w_down=s_d, shared_h=sh_h,
                               shared_y=sh_y)
            torch.cuda.synchronize()
            outs.append([t.view(torch.int16 if dtype == torch.bfloat16 else torch.int32).cpu()
                         for t in (h, y, sh_h, sh_y)])
    finally:
        moe.moe_set_gemm_max_cus(0)
    assert not torch.isnan(outs[0][1].view(dtype)).any()
    for other in outs[1:]:
        for a, b in zip(outs[0], other):
            assert torch.equal(a, b)
