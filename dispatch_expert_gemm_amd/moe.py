"""Thin Python binding of libmoe.so (argument marshalling only).

Every function has the name of the C entry point it calls and takes torch CUDA tensors; the work
runs in the library's HIP kernels on the current torch stream. There is no fallback: if the
library is missing, or returns an error, a RuntimeError is raised.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

# the in-tree build; MOE_LIBRARY may name another build of the same sources (e.g. a tuning variant)
LIB_PATH = os.environ.get("MOE_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

MOE_F32, MOE_BF16 = 0, 1
GATES = {"softmax": 0, "sigmoid": 1}
LAYOUT_FIELDS = ("expert_counts", "expert_offsets", "group_expert", "group_offsets",
                 "rank_counts", "rank_offsets", "send_counts", "row_of_slot", "slot_of_row",
                 "pair_counts", "pair_offsets", "pair_token", "pair_of_slot", "pair_send_counts",
                 "expand_src")

_P = ctypes.c_void_p
_I = ctypes.c_int


class Shape(ctypes.Structure):
    _fields_ = [("N", _I), ("E", _I), ("k", _I), ("W", _I), ("H", _I)]


class _LayoutC(ctypes.Structure):
    _fields_ = [(f, _P) for f in LAYOUT_FIELDS]


_lib = None


def lib():
    """The loaded libmoe.so (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m dispatch_expert_gemm_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        sig = {
            "moe_route": [_P, _P, _I, _I, _I, _I, _P, _P, _P, _I, _P, _P],
            "moe_gate_route": [_P, _I, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _I, _P,
                               _P],
            "moe_gate_workspace_bytes": [_I, _I],
            "moe_gate_prepare": [_P, _I, _I, _P, _P],
            "moe_shuffle_fit": [_P, _P, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P],
            "moe_shuffle_fit_workspace_bytes": [_I, _I],
            "moe_shuffle_plan": [_P, _P, _I, _I, _I, _I, _P, _P, _P, ctypes.c_float,
                                 ctypes.c_float, _P, _P, _P, _P, _P, _P, _P],
            "moe_shuffle_plan_workspace_bytes": [_I],
            "moe_device_info": [_P, _P, _P, _P],
            "moe_dispatch_layout": [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _P, _P],
            "moe_dispatch_layout_noalloc": [_P, _P, _P, _P, _P, _I, _I, _I, _P, _P],
            "moe_expert_ffn": [_P, _P, _I, _P, _P, _I, _P, _P, _I, _I, _I, _P, _P, _I, _I, _P,
                               _I, _P, _P, _P, _P, _I, _I, _P],
            "moe_pack_weights": [_P, _I, _I, _I, _I, _P, _P],
            "moe_set_gemm_max_cus": [_I],
            "moe_layer_fused": [_P, _I, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _I, _P, _P, _I,
                                _P, _P, _P, _P, _P],
            "moe_layer_fused_workspace_bytes": [_I, _I, _I, _I, _I, _I],
            "moe_combine": [_P, _P, _I, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _I, _P, _P,
                            _P],
            "moe_coselect_counts": [_P, _I, _I, _I, _P, _P],
            "moe_placement_partition": [_P, _I, _I, _I, _P, _P],
            "moe_layout_bytes": [_P],
            "moe_layout_carve": [_P, _P, _P],
            "moe_layout_workspace_bytes": [_P],
            "moe_status_string": [_I],
            "moe_last_error": [],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = _I
        L.moe_layout_bytes.restype = ctypes.c_size_t
        L.moe_layout_workspace_bytes.restype = ctypes.c_size_t
        L.moe_gate_workspace_bytes.restype = ctypes.c_size_t
        L.moe_shuffle_fit_workspace_bytes.restype = ctypes.c_size_t
        L.moe_shuffle_plan_workspace_bytes.restype = ctypes.c_size_t
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(status: int, what: str):
    if status != 0:
        L = lib()
        raise RuntimeError(f"{what}: {L.moe_status_string(status).decode()} "
                           f"({L.moe_last_error().decode()})")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dtypes(want, *ts):
    """Every given tensor has dtype `want` (a torch dtype, or None: all the same float type)."""
    given = [t for t in ts if isinstance(t, torch.Tensor)]
    if not given:
        return
    want = want or given[0].dtype
    for t in given:
        if t.dtype != want:
            raise TypeError(f"expected {want} tensors, got {t.dtype}")


def _dev(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda or not t.is_contiguous():
                raise ValueError("tensors must be contiguous CUDA tensors")


class Layout:
    """Caller-owned layout arrays: one int32 device buffer carved by moe_layout_carve."""

    def __init__(self, N, E, k, W, H, device="cuda"):
        self.shape = Shape(N, E, k, W, H)
        L = lib()
        nbytes = L.moe_layout_bytes(ctypes.byref(self.shape))
        if nbytes == 0:
            raise ValueError("invalid layout shape")
        self.buf = torch.empty(nbytes // 4, dtype=torch.int32, device=device)
        self.c = _LayoutC()
        _check(L.moe_layout_carve(ctypes.byref(self.shape), _ptr(self.buf), ctypes.byref(self.c)),
               "moe_layout_carve")
        self.ws = torch.empty(max(1, L.moe_layout_workspace_bytes(ctypes.byref(self.shape))),
                              dtype=torch.uint8, device=device)
        kw = min(k, W)
        self._len = dict(expert_counts=E, expert_offsets=E, group_expert=E, group_offsets=E + 1,
                         rank_counts=W, rank_offsets=W + 1, send_counts=W * W, row_of_slot=N * k,
                         slot_of_row=N * k, pair_counts=W, pair_offsets=W + 1,
                         pair_token=N * kw, pair_of_slot=N * k, pair_send_counts=W * W,
                         expand_src=N * k)

    def __getitem__(self, name) -> torch.Tensor:
        """A torch view of one layout array."""
        off = (getattr(self.c, name) - self.buf.data_ptr()) // 4
        return self.buf[off:off + self._len[name]]

    def ptr(self, name, offset=0):
        return ctypes.c_void_p(getattr(self.c, name) + 4 * offset)


def _count_args(counts, N, E):
    """counts = (layout, expert_rank or None): the route also writes layout.ws's count rows."""
    if counts is None:
        return None, 0, None
    layout, expert_rank = counts
    _dtypes(torch.int32, expert_rank)
    _dev(expert_rank)
    if (layout.shape.N, layout.shape.E) != (N, E):
        raise ValueError(f"the layout is for N={layout.shape.N}, E={layout.shape.E}, "
                         f"the route for N={N}, E={E}")
    return expert_rank, layout.shape.W, layout.ws


def moe_route(logits, bias, k, gate="softmax", topk_idx=None, topk_w=None, counts=None):
    """counts = (layout, expert_rank): also write the count rows of layout.ws, so a following
    moe_dispatch_layout(layout, ..., counts_ready=True) skips its count step."""
    _dtypes(torch.float32, logits, bias, topk_w)
    _dtypes(torch.int32, topk_idx)
    _dev(logits, bias)
    N, E = logits.shape
    pl, W, ws = _count_args(counts, N, E)
    if topk_idx is None:
        topk_idx = torch.empty((N, k), dtype=torch.int32, device=logits.device)
    if topk_w is None:
        topk_w = torch.empty((N, k), dtype=torch.float32, device=logits.device)
    _check(lib().moe_route(_ptr(logits), _ptr(bias), N, E, k, GATES[gate], _ptr(topk_idx),
                           _ptr(topk_w), _ptr(pl), W, _ptr(ws), _stream()), "moe_route")
    return topk_idx, topk_w


def moe_gate_prepare(w_router, workspace=None):
    """The split of W_R the gate multiplies with, once; returns the workspace that
    moe_gate_route(..., workspace=ws, prepared=True) then uses."""
    _dtypes(torch.float32, w_router)
    _dev(w_router, workspace)
    E, H = w_router.shape
    need = lib().moe_gate_workspace_bytes(E, H)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=w_router.device)
    elif workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace holds fewer than the {need} bytes the split needs")
    _check(lib().moe_gate_prepare(_ptr(w_router), E, H, _ptr(workspace), _stream()),
           "moe_gate_prepare")
    return workspace


def moe_gate_route(x, w_router, bias, k, gate="softmax", logits=None, topk_idx=None,
                   topk_w=None, workspace=None, counts=None, prepared=False):
    """Router linear layer on the device (logits = x W_R^T, fp32) followed by moe_route.
    counts: as for moe_route. prepared: `workspace` holds moe_gate_prepare's split of w_router
    (w_router then only gives the shape)."""
    _dtypes(torch.float32, w_router, bias, logits, topk_w)
    _dtypes(torch.int32, topk_idx)
    _dev(x, w_router, bias, logits, workspace)
    N, H = x.shape
    E = w_router.shape[0]
    if tuple(w_router.shape) != (E, H):
        raise ValueError(f"w_router must be [E, {H}], got {tuple(w_router.shape)}")
    pl, W, lws = _count_args(counts, N, E)
    if prepared and workspace is None:
        raise ValueError("prepared=True needs the workspace moe_gate_prepare wrote")
    need = lib().moe_gate_workspace_bytes(E, H)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    elif workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace holds fewer than the {need} bytes moe_gate_route needs")
    for name, t, shape in (("logits", logits, (N, E)), ("topk_idx", topk_idx, (N, k)),
                           ("topk_w", topk_w, (N, k)), ("bias", bias, (E,))):
        if t is not None and tuple(t.shape) != shape:
            raise ValueError(f"{name} must be {shape}, got {tuple(t.shape)}")
    if logits is None:
        logits = torch.empty((N, E), dtype=torch.float32, device=x.device)
    if topk_idx is None:
        topk_idx = torch.empty((N, k), dtype=torch.int32, device=x.device)
    if topk_w is None:
        topk_w = torch.empty((N, k), dtype=torch.float32, device=x.device)
    _check(lib().moe_gate_route(_ptr(x), _dtype_code(x), None if prepared else _ptr(w_router),
                                _ptr(bias), N, H, E, k,
                                GATES[gate], _ptr(workspace), _ptr(logits), _ptr(topk_idx),
                                _ptr(topk_w), _ptr(pl), W, _ptr(lws), _stream()),
           "moe_gate_route")
    return logits, topk_idx, topk_w


def moe_dispatch_layout(layout: Layout, topk_idx, expert_rank=None, x=None, dedup=False,
                        dst_rank=-1, rows_out=None, counts_ready=False):
    """counts_ready: layout.ws already holds the count rows (moe_route / moe_gate_route with
    counts=(layout, expert_rank) on the same topk_idx), so the count step is skipped."""
    _dtypes(torch.int32, topk_idx, expert_rank)
    _dtypes(None, x, rows_out)
    _dev(topk_idx, expert_rank, x, rows_out)
    dt = _dtype_code(x) if x is not None else MOE_F32
    _check(lib().moe_dispatch_layout(ctypes.byref(layout.shape), _ptr(topk_idx),
                                     _ptr(expert_rank), ctypes.byref(layout.c),
                                     _ptr(layout.ws), _ptr(x), dt, int(dedup), dst_rank,
                                     int(bool(counts_ready)), _ptr(rows_out), _stream()),
           "moe_dispatch_layout")
    return rows_out


def moe_dispatch_layout_noalloc(layout: Layout, topk_idx, expert_rank=None, x=None, dedup=False,
                                dst_rank=-1, rows_out=None):
    """moe_dispatch_layout with the library's fixed scratch array as its workspace (the call
    allocates nothing; layout.ws is not used)."""
    _dtypes(torch.int32, topk_idx, expert_rank)
    _dtypes(None, x, rows_out)
    _dev(topk_idx, expert_rank, x, rows_out)
    dt = _dtype_code(x) if x is not None else MOE_F32
    _check(lib().moe_dispatch_layout_noalloc(ctypes.byref(layout.shape), _ptr(topk_idx),
                                             _ptr(expert_rank), ctypes.byref(layout.c), _ptr(x),
                                             dt, int(dedup), dst_rank, _ptr(rows_out),
                                             _stream()), "moe_dispatch_layout_noalloc")
    return rows_out


def moe_expert_ffn(rows, group_offsets, G, w_gate_up, w_down, h, y, max_rows, row_gather=None,
                   gather_base=None, shared_x=None, shared_w_gate_up=None, shared_w_down=None,
                   shared_h=None, shared_y=None, phases=3, y_absolute=False,
                   weights_packed=False):
    """group_offsets / row_gather / gather_base: torch int32 views or ctypes pointers.
    phases: 1 = gate/up GEMM only, 2 = down GEMM only, 3 = both.
    y_absolute: y is indexed by absolute row (a group_offsets value).
    weights_packed: the four weight tensors came from moe_pack_weights."""
    ref = rows if rows is not None else shared_x
    _dtypes(None, rows, w_gate_up, w_down, h, y, shared_x, shared_w_gate_up, shared_w_down,
            shared_h, shared_y)
    _dtypes(torch.int32, group_offsets, row_gather, gather_base)
    _dev(rows, w_gate_up, w_down, h, y, shared_x, shared_w_gate_up, shared_w_down, shared_h,
         shared_y)
    H = ref.shape[-1]
    wgu = w_gate_up if w_gate_up is not None else shared_w_gate_up
    I = wgu.shape[-2] // 2
    S = 0 if shared_w_gate_up is None else shared_w_gate_up.shape[0]
    M_sh = 0 if shared_x is None else shared_x.shape[0]
    as_p = lambda t: t if isinstance(t, ctypes.c_void_p) else _ptr(t)
    _check(lib().moe_expert_ffn(_ptr(rows), as_p(group_offsets), G, as_p(row_gather),
                                as_p(gather_base), max_rows, _ptr(w_gate_up), _ptr(w_down), H, I,
                                _dtype_code(ref), _ptr(h), _ptr(y), int(bool(y_absolute)), S,
                                _ptr(shared_x), M_sh,
                                _ptr(shared_w_gate_up), _ptr(shared_w_down), _ptr(shared_h),
                                _ptr(shared_y), phases, int(bool(weights_packed)),
                                _stream()), "moe_expert_ffn")
    return y


def moe_pack_weights(w, NB, out=None):
    """Packed copy of bf16 expert weights [G, NB * Nn, K] (same shape and dtype, permuted)."""
    _dtypes(torch.bfloat16, w, out)
    _dev(w, out)
    G, R, K = w.shape
    if out is None:
        out = torch.empty_like(w)
    _check(lib().moe_pack_weights(_ptr(w), G, NB, R // NB, K, _ptr(out), _stream()),
           "moe_pack_weights")
    return out


def moe_combine(layout: Layout, y, topk_idx, topk_w, out, expert_rank=None, dedup=False,
                t_begin=0, t_end=None, shared=None, partial=None, y_is_pair_rows=False,
                dst_rank=-1):
    """dst_rank (dedup only): -1 = partials of every pair row; r = rank r's pair rows only."""
    _dtypes(None, y, out, shared, partial)
    _dtypes(torch.int32, topk_idx, expert_rank)
    _dtypes(torch.float32, topk_w)
    _dev(y, topk_idx, topk_w, out, expert_rank, shared, partial)
    t_end = layout.shape.N if t_end is None else t_end
    n_shared = 0 if shared is None else shared.shape[0]
    _check(lib().moe_combine(ctypes.byref(layout.shape), _ptr(y), int(y_is_pair_rows),
                             ctypes.byref(layout.c), _ptr(topk_idx), _ptr(topk_w),
                             _ptr(expert_rank), _dtype_code(y), int(dedup), int(dst_rank),
                             t_begin, t_end,
                             _ptr(shared), n_shared, _ptr(partial), _ptr(out), _stream()),
           "moe_combine")
    return out


def moe_coselect_counts(topk_idx, E, counts=None):
    _dtypes(torch.int32, topk_idx, counts)
    _dev(topk_idx)
    N, k = topk_idx.shape
    if counts is None:
        counts = torch.empty((E, E), dtype=torch.int32, device=topk_idx.device)
    _check(lib().moe_coselect_counts(_ptr(topk_idx), N, E, k, _ptr(counts), _stream()),
           "moe_coselect_counts")
    return counts


def moe_placement_partition(counts, G, i_max=0):
    """Host call: counts is an [E, E] integer array (numpy or CPU tensor)."""
    c = np.ascontiguousarray(np.asarray(counts), dtype=np.int64)
    E = c.shape[0]
    group = np.empty(E, np.int32)
    swaps = ctypes.c_int(0)
    _check(lib().moe_placement_partition(c.ctypes.data_as(_P), E, G, i_max,
                                         group.ctypes.data_as(_P), ctypes.byref(swaps)),
           "moe_placement_partition")
    return group, swaps.value


def moe_shuffle_fit(prev2, prev1, cur, placement, E, P, workspace=None):
    """Token-shuffle tables (F [E, P], S [E, E, P] float32, n [E, E] int32) from one trace."""
    _dtypes(torch.int32, prev2, prev1, cur, placement)
    _dev(prev2, prev1, cur, placement, workspace)
    T, k = cur.shape
    dev = cur.device
    if workspace is None:
        workspace = torch.empty(lib().moe_shuffle_fit_workspace_bytes(E, P), dtype=torch.uint8,
                                device=dev)
    F = torch.empty((E, P), dtype=torch.float32, device=dev)
    S = torch.empty((E, E, P), dtype=torch.float32, device=dev)
    n = torch.empty((E, E), dtype=torch.int32, device=dev)
    _check(lib().moe_shuffle_fit(_ptr(prev2), _ptr(prev1), _ptr(cur), T, k, E, P,
                                 _ptr(placement), _ptr(workspace), _ptr(F), _ptr(S), _ptr(n),
                                 _stream()), "moe_shuffle_fit")
    return F, S, n


def moe_shuffle_plan(prev2, prev1, F, S, n, beta, w_max, workspace=None, out=None):
    """Owner ranks and owner-major order of the tokens; returns (d, conf, owner, order, inverse).
    `out` may pass those five tensors preallocated."""
    _dtypes(torch.int32, prev2, prev1, n)
    _dtypes(torch.float32, F, S)
    _dev(prev2, prev1, F, S, n, workspace)
    T, k = prev1.shape
    E, P = F.shape
    dev = prev1.device
    if workspace is None:
        workspace = torch.empty(max(1, lib().moe_shuffle_plan_workspace_bytes(T)),
                                dtype=torch.uint8, device=dev)
    if out is None:
        out = (torch.empty((T, P), dtype=torch.float32, device=dev),
               torch.empty(T, dtype=torch.float32, device=dev),
               torch.empty(T, dtype=torch.int32, device=dev),
               torch.empty(T, dtype=torch.int32, device=dev),
               torch.empty(T, dtype=torch.int32, device=dev))
    d, conf, owner, order, inverse = out
    _check(lib().moe_shuffle_plan(_ptr(prev2), _ptr(prev1), T, k, E, P, _ptr(F), _ptr(S),
                                  _ptr(n), float(beta), float(w_max), _ptr(workspace), _ptr(d),
                                  _ptr(conf), _ptr(owner), _ptr(order), _ptr(inverse),
                                  _stream()), "moe_shuffle_plan")
    return d, conf, owner, order, inverse


def moe_set_gemm_max_cus(n: int):
    """Caps the grouped GEMM's persistent grid at n compute units (0 = all); process-wide."""
    _check(lib().moe_set_gemm_max_cus(int(n)), "moe_set_gemm_max_cus")


def moe_device_info():
    """(compute units, LDS bytes per CU, peak shader clock kHz, memory clock kHz) of the current
    device."""
    v = [ctypes.c_int(0) for _ in range(4)]
    _check(lib().moe_device_info(*[ctypes.byref(x) for x in v]), "moe_device_info")
    return tuple(x.value for x in v)


def moe_layer_fused(x, logits, bias, k, gate, w_gate_up, w_down, shared_w_gate_up=None,
                    shared_w_down=None, workspace=None, out=None, topk_idx=None, topk_w=None,
                    weights_packed=False):
    """The whole layer in one launch for small batches. weights_packed: the four weight tensors
    came from moe_pack_weights (bf16). The workspace's first 4 KB are the launch's device-wide
    counters: a new workspace is zeroed; every call leaves them at zero unless a stage wait gave
    up (fused_error reports it)."""
    _dtypes(torch.float32, logits, bias, topk_w)
    _dtypes(torch.int32, topk_idx)
    _dtypes(None, x, w_gate_up, w_down, shared_w_gate_up, shared_w_down, out)
    _dev(x, logits, bias, w_gate_up, w_down, shared_w_gate_up, shared_w_down, workspace, out)
    N, H = x.shape
    E = logits.shape[1]
    I = w_gate_up.shape[1] // 2
    S = 0 if shared_w_gate_up is None else shared_w_gate_up.shape[0]
    dt = _dtype_code(x)
    if tuple(logits.shape) != (N, E) or tuple(w_gate_up.shape) != (E, 2 * I, H) or \
            tuple(w_down.shape) != (E, H, I) or (S and (
                tuple(shared_w_gate_up.shape) != (S, 2 * I, H) or
                tuple(shared_w_down.shape) != (S, H, I))):
        raise ValueError("moe_layer_fused: logits [N, E], w_gate_up [E, 2I, H], w_down [E, H, I] "
                         "and shared weights [S, 2I, H], [S, H, I] expected")
    need = lib().moe_layer_fused_workspace_bytes(N, H, k, I, S, dt)
    if workspace is None:
        workspace = torch.zeros(max(need, 4096), dtype=torch.uint8, device=x.device)
    elif workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace holds fewer than the {need} bytes moe_layer_fused needs")
    if out is None:
        out = torch.empty_like(x)
    if topk_idx is None:
        topk_idx = torch.empty((N, k), dtype=torch.int32, device=x.device)
    if topk_w is None:
        topk_w = torch.empty((N, k), dtype=torch.float32, device=x.device)
    _check(lib().moe_layer_fused(_ptr(x), dt, _ptr(logits), _ptr(bias), N, H, E, k, GATES[gate],
                                 I, _ptr(w_gate_up), _ptr(w_down), S, _ptr(shared_w_gate_up),
                                 _ptr(shared_w_down), int(bool(weights_packed)), _ptr(topk_idx),
                                 _ptr(topk_w),
                                 _ptr(workspace), _ptr(out), _stream()), "moe_layer_fused")
    return out, topk_idx, topk_w, workspace


def fused_error(workspace) -> int:
    """The fused layer's error flag (nonzero: a stage wait gave up and the outputs are
    undefined). Synchronises the device."""
    torch.cuda.synchronize()
    return int(workspace[:4096].view(torch.int32)[32 * 18].item())

