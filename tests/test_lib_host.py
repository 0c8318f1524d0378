"""CPU checks of libmoe.so: it loads, exports every function include/moe.h declares, and its host
functions (layout sizing and carving, the Algorithm 1 partition, argument checks that reject bad
calls before any launch) behave as documented. No GPU work is issued here."""
import ctypes
import os
import re

import numpy as np
import pytest

from dispatch_expert_gemm_amd import moe
from oracle import moe_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(moe.LIB_PATH):
        from dispatch_expert_gemm_amd import build
        build.build()
    return moe.lib()


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert len(names) >= 11
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    assert L.moe_status_string(0) == b"MOE_OK"
    assert b"EINVAL" in L.moe_status_string(1)


def test_layout_sizes_and_carve(L):
    s = moe.Shape(4096, 64, 6, 8, 2048)
    nb = L.moe_layout_bytes(ctypes.byref(s))
    assert nb > 0 and nb % 256 == 0
    base = 1 << 20
    c = moe._LayoutC()
    assert L.moe_layout_carve(ctypes.byref(s), ctypes.c_void_p(base), ctypes.byref(c)) == 0
    ptrs = [getattr(c, f) for f in moe.LAYOUT_FIELDS]
    assert ptrs == sorted(ptrs) and all(p % 256 == 0 for p in ptrs)
    assert ptrs[-1] + 4 * 4096 * 6 <= base + nb
    assert L.moe_layout_workspace_bytes(ctypes.byref(s)) >= 16 * (64 + 8) * 4
    bad = moe.Shape(4096, 63, 6, 8, 2048)          # E not a multiple of W
    assert L.moe_layout_bytes(ctypes.byref(bad)) == 0


@pytest.mark.parametrize("E,G,seed", [(8, 2, 0), (12, 3, 1), (16, 4, 2), (64, 32, 3)])
def test_partition_matches_oracle(L, E, G, seed):
    rng = np.random.default_rng(seed)
    idx = rng.integers(0, E, size=(3000, 2))
    idx = idx[idx[:, 0] != idx[:, 1]].astype(np.int32)
    Wc = O.coselect_counts(idx, E)
    want, wsw = O.partition(Wc, G)
    got, gsw = moe.moe_placement_partition(Wc, G)
    assert np.array_equal(got, want) and gsw == wsw
    got1, s1 = moe.moe_placement_partition(Wc, G, i_max=1)
    want1, _ = O.partition(Wc, G, i_max=1)
    assert np.array_equal(got1, want1) and s1 == min(1, wsw)


def test_argument_checks_reject_before_launch(L):
    P = ctypes.c_void_p
    fake = P(1 << 20)
    # k > E, E too large, gate unknown
    assert L.moe_route(fake, None, 16, 8, 9, 0, fake, fake, None, 0, None, None) == 1
    assert L.moe_route(fake, None, 16, 1024, 2, 0, fake, fake, None, 0, None, None) == 1
    assert L.moe_route(fake, None, 16, 8, 2, 7, fake, fake, None, 0, None, None) == 1
    assert L.moe_route(None, None, 0, 8, 2, 0, None, None, None, 0, None, None) == 0  # N = 0
    assert b"moe_route" in L.moe_last_error()
    # count rows requested with an invalid W: 0, above 64, not dividing E, not dividing N
    for W in (0, 65, 3):
        assert L.moe_route(fake, None, 48, 8, 2, 0, fake, fake, None, W, fake, None) == 1
    assert L.moe_route(fake, None, 18, 8, 2, 0, fake, fake, None, 4, fake, None) == 1
    assert b"layout workspace" in L.moe_last_error()
    assert L.moe_gate_route(fake, 1, fake, None, 16, 128, 8, 2, 0, fake, fake, fake, fake,
                            None, 3, fake, None) == 1
    s = moe.Shape(16, 8, 2, 4, 128)
    lay = moe._LayoutC()
    assert L.moe_dispatch_layout(ctypes.byref(s), fake, None, ctypes.byref(lay), fake, None, 0,
                                 0, 4, 0, None, None) == 1     # dst_rank out of range
    bad = moe.Shape(15, 8, 2, 4, 128)                           # N not a multiple of W
    assert L.moe_dispatch_layout(ctypes.byref(bad), fake, None, ctypes.byref(lay), fake, None, 0,
                                 0, -1, 0, None, None) == 1
    # ffn: bf16 H not a multiple of 128
    assert L.moe_expert_ffn(fake, fake, 4, None, None, 64, fake, fake, 100, 256, 1, fake, fake, 0,
                            0, None, 0, None, None, None, None, 3, 0, None) == 1
    assert L.moe_expert_ffn(fake, fake, 4, None, None, 64, fake, fake, 128, 256, 1, fake, fake, 0,
                            0, None, 0, None, None, None, None, 0, 0, None) == 1   # no phase
    # ffn: bf16 operand blocks addressed with 32-bit byte offsets must stay below 4 GiB
    rows_4g = (1 << 32) // (2 * 4096)                            # rows x H x 2 bytes = 4 GiB
    assert L.moe_expert_ffn(fake, fake, 4, None, None, rows_4g, fake, fake, 4096, 1024, 1, fake,
                            fake, 0, 0, None, 0, None, None, None, None, 3, 0, None) == 1
    assert b"4 GiB" in L.moe_last_error()
    assert L.moe_expert_ffn(fake, fake, 4, None, None, 64, fake, fake, 4096, 1024, 1, fake, fake,
                            0, 1, fake, rows_4g, fake, fake, fake, fake, 3, 0, None) == 1
    assert L.moe_expert_ffn(fake, fake, 1, None, None, 64, fake, fake, 32768, 32768, 1, fake, fake,
                            0, 0, None, 0, None, None, None, None, 3, 0, None) == 1  # 4 I H bytes
    # combine: t_end > N
    assert L.moe_combine(ctypes.byref(s), fake, 0, ctypes.byref(lay), fake, fake, None, 0, 0, -1,
                         0, 17, None, 0, None, fake, None) == 1
    # combine: dst_rank outside [-1, W)
    assert L.moe_combine(ctypes.byref(s), fake, 0, ctypes.byref(lay), fake, fake, None, 0, 1, 4,
                         0, 16, None, 0, fake, fake, None) == 1
    assert L.moe_coselect_counts(fake, 4, 8, 9, fake, None) == 1
    # shuffle planner: T not a multiple of P, P > 64, beta < 0, w_max > 1, k = 0
    f32 = ctypes.c_float
    assert L.moe_shuffle_plan(fake, fake, 10, 2, 8, 4, fake, fake, fake, f32(1), f32(0.5), fake,
                              fake, fake, fake, fake, fake, None) == 1
    assert L.moe_shuffle_plan(fake, fake, 128, 2, 8, 128, fake, fake, fake, f32(1), f32(0.5),
                              fake, fake, fake, fake, fake, fake, None) == 1
    assert L.moe_shuffle_plan(fake, fake, 8, 2, 8, 4, fake, fake, fake, f32(-1), f32(0.5), fake,
                              fake, fake, fake, fake, fake, None) == 1
    assert L.moe_shuffle_plan(fake, fake, 8, 2, 8, 4, fake, fake, fake, f32(1), f32(1.5), fake,
                              fake, fake, fake, fake, fake, None) == 1
    assert L.moe_shuffle_plan(None, None, 0, 2, 8, 4, None, None, None, f32(1), f32(0.5), None,
                              None, None, None, None, None, None) == 0    # T = 0: nothing to do
    assert L.moe_shuffle_fit(fake, fake, fake, 16, 0, 8, 4, fake, fake, fake, fake, fake,
                             None) == 1
    assert L.moe_shuffle_fit(fake, fake, fake, 16, 2, 8, 4, None, fake, fake, fake, fake,
                             None) == 1                                 # no placement
    assert L.moe_shuffle_fit_workspace_bytes(128, 8) == 128 * 8 * 4 + 128 * 128 * 8 * 4
    assert L.moe_shuffle_plan_workspace_bytes(1000) == 4 * 4096
    assert L.moe_placement_partition(None, 8, 3, 0, None, None) == 1


def test_gate_route_argument_checks(L):
    P = ctypes.c_void_p
    fake = P(1 << 20)
    # H not a multiple of 32, E above 256, k > E, unknown dtype, NULL logits, NULL workspace
    def gate(*a):   # no count rows: expert_rank NULL, W 0, layout workspace NULL, null stream
        return L.moe_gate_route(*a, None, 0, None, None)
    assert gate(fake, 1, fake, None, 16, 100, 8, 2, 0, fake, fake, fake, fake) == 1
    assert gate(fake, 1, fake, None, 16, 128, 300, 2, 0, fake, fake, fake, fake) == 1
    assert gate(fake, 1, fake, None, 16, 128, 8, 9, 0, fake, fake, fake, fake) == 1
    assert gate(fake, 5, fake, None, 16, 128, 8, 2, 0, fake, fake, fake, fake) == 1
    assert gate(fake, 1, fake, None, 16, 128, 8, 2, 0, fake, None, fake, fake) == 1
    assert gate(fake, 1, fake, None, 16, 128, 8, 2, 0, None, fake, fake, fake) == 1
    assert b"moe_gate_route" in L.moe_last_error()
    assert gate(None, 1, None, None, 0, 128, 8, 2, 0, None, None, None, None) == 0
    assert L.moe_gate_workspace_bytes(256, 7168) == 256 * 7168 * 4
    # the one-time split: E above 256, H not a multiple of 32, NULL weights or workspace
    assert L.moe_gate_prepare(fake, 300, 128, fake, None) == 1
    assert L.moe_gate_prepare(fake, 8, 100, fake, None) == 1
    assert L.moe_gate_prepare(None, 8, 128, fake, None) == 1
    assert L.moe_gate_prepare(fake, 8, 128, None, None) == 1
    assert b"moe_gate_prepare" in L.moe_last_error()


def test_ffn_row_limit_at_the_largest_hidden_size(L):
    # the host accepts (max_rows + 1) x H x 2 bytes up to 2^32 - 1 (the GPU test runs that many
    # rows) and rejects one row more before any launch
    P = ctypes.c_void_p
    fake = P(1 << 20)
    H, I = 7168, 256
    ok_rows = (2 ** 32 - 1) // (2 * H) - 1
    assert (ok_rows + 1) * H * 2 <= 2 ** 32 - 1 < (ok_rows + 2) * H * 2
    assert L.moe_expert_ffn(fake, fake, 2, None, None, ok_rows + 1, fake, fake, H, I, 1, fake,
                            fake, 0, 0, None, 0, None, None, None, None, 1, 0, None) == 1
    assert b"4 GiB" in L.moe_last_error()
    assert L.moe_expert_ffn(fake, fake, 2, None, None, 64, fake, fake, H, I, 1, fake, fake, 0, 1,
                            fake, ok_rows + 1, fake, fake, fake, fake, 1, 0, None) == 1
    assert b"4 GiB" in L.moe_last_error()


def test_binding_rejects_mixed_dtypes():
    # the binding passes one dtype code per call: operands of another type are refused before
    # anything reaches the library
    import torch
    f32 = torch.zeros((4, 8), dtype=torch.float32)
    bf = torch.zeros((4, 8), dtype=torch.bfloat16)
    i64 = torch.zeros((4, 2), dtype=torch.int64)
    with pytest.raises(TypeError):
        moe.moe_route(bf, None, 2)
    with pytest.raises(TypeError):
        moe.moe_route(f32, None, 2, topk_idx=i64)
    with pytest.raises(TypeError):
        moe.moe_expert_ffn(bf, None, 1, f32, bf, bf, bf, 4)
    with pytest.raises(TypeError):
        moe.moe_coselect_counts(i64, 8)


def test_empty_inputs_launch_nothing(L):
    # zero tokens, an empty owned range or an empty trace: every call returns OK at once (no
    # device pointer is touched, so NULLs and placeholders are fine)
    P = ctypes.c_void_p
    fake = P(1 << 20)
    s0 = moe.Shape(0, 8, 2, 4, 128)
    lay = moe._LayoutC()
    assert L.moe_dispatch_layout(ctypes.byref(s0), None, None, ctypes.byref(lay), None, None, 0,
                                 0, -1, 1, None, None) == 0
    s = moe.Shape(16, 8, 2, 4, 128)
    for f in moe.LAYOUT_FIELDS:
        setattr(lay, f, fake.value)
    assert L.moe_combine(ctypes.byref(s), fake, 0, ctypes.byref(lay), fake, fake, None, 1, 0, -1,
                         5, 5, None, 0, None, fake, None) == 0           # t_begin == t_end
    assert L.moe_shuffle_plan(None, None, 0, 2, 8, 4, fake, fake, fake, 1.0, 0.5, None, None,
                              None, None, None, None, None) == 0      # T = 0


def test_noalloc_rejects_oversized_layouts(L):
    # the fixed scratch array bounds the layout's count rows: a shape that needs more is refused
    # on the host before anything touches a device; the largest shape at E = 512, W = 64 fits
    fake = ctypes.c_void_p(1 << 20)
    s = moe.Shape(116480 + 64, 512, 8, 64, 128)
    assert L.moe_layout_workspace_bytes(ctypes.byref(s)) > 16 << 20
    assert L.moe_layout_workspace_bytes(ctypes.byref(moe.Shape(116480, 512, 8, 64, 128))) <= 16 << 20
    lay = moe._LayoutC()
    assert L.moe_dispatch_layout_noalloc(ctypes.byref(s), fake, None, ctypes.byref(lay), None, 0,
                                         0, -1, None, None) == 1
    assert b"scratch" in L.moe_last_error()
    s0 = moe.Shape(0, 8, 2, 4, 128)                               # N = 0: nothing to do
    assert L.moe_dispatch_layout_noalloc(ctypes.byref(s0), None, None, ctypes.byref(lay), None,
                                         0, 0, -1, None, None) == 0


def test_pack_weights_argument_checks(L):
    fake = ctypes.c_void_p(1 << 20)
    other = ctypes.c_void_p(1 << 21)
    assert L.moe_pack_weights(fake, 2, 3, 128, 128, other, None) == 1      # NB not 1 or 2
    assert L.moe_pack_weights(fake, 2, 2, 64, 128, other, None) == 1       # gate/up Nn % 128
    assert L.moe_pack_weights(fake, 2, 1, 128, 128, other, None) == 1      # down Nn % 256
    assert L.moe_pack_weights(fake, 2, 1, 256, 96, other, None) == 1       # K % 64
    assert L.moe_pack_weights(fake, 2, 1, 256, 128, fake, None) == 1       # in place
    assert L.moe_pack_weights(None, 0, 1, 256, 128, None, None) == 0       # nothing to do
    # the FFN refuses packed weights where the packed panels do not tile H and I
    assert L.moe_expert_ffn(fake, fake, 2, None, None, 64, fake, fake, 384, 256, 1, fake, fake,
                            0, 0, None, 0, None, None, None, None, 3, 1, None) == 1
    assert b"packed" in L.moe_last_error()


def test_gate_route_rejects_32bit_offset_overflow(L):
    fake = ctypes.c_void_p(1 << 20)
    # 256 experts x H x 4 bytes of router weights reach 4 GiB: refused before any launch
    H = (1 << 32) // (4 * 256)
    assert L.moe_gate_route(fake, 1, fake, None, 16, H, 256, 2, 0, fake, fake, fake, fake,
                            None, 0, None, None) == 1
    assert b"4 GiB" in L.moe_last_error()


@pytest.mark.parametrize("E,G", [(128, 8), (256, 16), (512, 32)])
def test_partition_matches_oracle_large(L, E, G):
    # Algorithm 1 on co-selection counts with a planted structure (blocks of experts that are
    # chosen together), at the expert counts of the pages' models and beyond
    rng = np.random.default_rng(E)
    blocks = rng.permutation(E).reshape(-1, E // G)
    Wc = rng.integers(0, 3, size=(E, E))
    for b in blocks:
        Wc[np.ix_(b, b)] += rng.integers(5, 40, size=(len(b), len(b)))
    Wc = np.triu(Wc, 1)
    Wc = (Wc + Wc.T).astype(np.int64)
    want, wsw = O.partition(Wc, G)
    got, gsw = moe.moe_placement_partition(Wc, G)
    assert np.array_equal(got, want) and gsw == wsw and wsw > 0


def test_layer_fused_argument_checks(L):
    fake = ctypes.c_void_p(1 << 20)

    def fused(N, H, E, k, I, S=0, dtype=1, gate=0):
        return L.moe_layer_fused(fake, dtype, fake, None, N, H, E, k, gate, I, fake, fake, S, fake,
                                 fake, 0, fake, fake, fake, fake, None)
    assert fused(1025, 128, 8, 1, 128) == 1        # more than 1024 tokens
    assert fused(1024, 128, 8, 5, 128) == 1        # N k above 4096 slots
    assert fused(64, 192, 8, 2, 128) == 1          # H not a multiple of 128
    assert fused(64, 128, 8, 2, 96) == 1           # I not a multiple of 128
    assert fused(64, 128, 8, 9, 128) == 1          # k > E
    assert fused(64, 128, 8, 2, 128, S=17) == 1    # too many shared experts
    assert fused(64, 128, 8, 2, 128, dtype=3) == 1
    assert fused(64, 128, 8, 2, 128, gate=4) == 1
    assert b"moe_layer_fused" in L.moe_last_error()
    assert L.moe_layer_fused(fake, 0, fake, None, 64, 256, 8, 2, 0, 128, fake, fake, 0, fake,
                             fake, 1, fake, fake, fake, fake, None) == 1   # packed needs bf16
    assert L.moe_layer_fused(fake, 1, fake, None, 64, 384, 8, 2, 0, 128, fake, fake, 0, fake,
                             fake, 1, fake, fake, fake, fake, None) == 1   # and H % 256
    assert L.moe_layer_fused(None, 1, None, None, 0, 128, 8, 2, 0, 128, None, None, 0, None, None,
                             0, None, None, None, None, None) == 0       # N = 0: nothing to do
    assert L.moe_layer_fused_workspace_bytes(64, 128, 2, 256, 1, 0) == \
        4096 + (64 * 2 + 64) * 256 * 4 + (64 * 2 + 64) * 128 * 4



def test_gemm_cu_cap_argument_check(L):
    assert L.moe_set_gemm_max_cus(-1) == 1          # MOE_EINVAL
    assert b"moe_set_gemm_max_cus" in L.moe_last_error()
    assert L.moe_set_gemm_max_cus(128) == 0
    assert L.moe_set_gemm_max_cus(0) == 0
