"""One MoE-layer step on one GPU: device buffers for a workload and the four library calls.

route -> dispatch layout (+ permute) -> grouped SwiGLU expert FFN (+ shared experts) -> combine,
enqueued on the current torch stream with no host synchronisation inside the step (optionally
the shared experts on a second stream; MicrobatchLayer pipelines microbatches of the batch over
three streams). Torch is only used to allocate and hold device memory and streams.

When a workload runs one rank's share (dst_rank = r), route and layout cover all N tokens, the
permute and the FFN only rank r's partition, and the combine rank r's owned tokens; the rows the
other ranks would return for those tokens are seeded stand-ins placed once at set-up (they are
not part of the step). With the deduplicating dispatcher the other ranks return one weighted
partial per (token, rank): set-up turns the stand-in rows into those partials once, and the
step's combine computes rank r's own partials (for every token it serves) and then sums each
owned token's partials.
"""
from __future__ import annotations

import numpy as np
import torch

from . import moe
from . import workloads as WL


class MoELayerRun:
    def __init__(self, w: WL.Workload, placement=None, device="cuda", inputs=None,
                 gen_threads=8, pack=None, inputs_packed=False):
        """placement: None (contiguous) or an [E] int array of expert ranks.
        inputs: optional dict of host tensors overriding the generated ones.
        pack: convert the bf16 expert weights to the packed layout once at set-up
        (moe_pack_weights; None = whenever the shapes allow it). inputs_packed: the expert and
        shared weights given in `inputs` are device tensors already packed."""
        self.w = w
        self.dev = torch.device(device)
        inputs = inputs or {}
        dt = w.torch_dtype
        N, E, k, W, H = w.N, w.E, w.k, w.W, w.H
        kw = min(k, W)
        self.e_loc = E // W

        self.host = {}

        def gen(name, fn):
            v = inputs[name] if name in inputs else fn()
            self.host[name] = v
            return v

        # inputs
        self.x = gen("x", lambda: WL.gen_x(w)).to(self.dev)
        self.logits = torch.from_numpy(np.asarray(gen("logits", lambda: WL.gen_logits(w)))).to(
            self.dev)
        b = gen("bias", lambda: WL.gen_bias(w))
        self.bias = None if b is None else torch.from_numpy(np.asarray(b)).to(self.dev)
        self.placement = None if placement is None else torch.as_tensor(
            np.asarray(placement, np.int32)).to(self.dev)
        self.swiglu = w.expert == "swiglu"
        if not self.swiglu and w.dst_rank >= 0:
            raise ValueError("identity experts run every rank's share (dst_rank = -1)")
        if self.swiglu:
            if w.dst_rank >= 0:
                if placement is not None:
                    raise ValueError("one rank's share needs the contiguous placement")
                self.local = list(range(w.dst_rank * self.e_loc, (w.dst_rank + 1) * self.e_loc))
            else:
                if placement is not None and not np.array_equal(
                        np.argsort(np.asarray(placement), kind="stable"), np.arange(E)):
                    raise ValueError("SwiGLU experts need weights stacked in group order; use "
                                     "the contiguous placement")
                self.local = list(range(E))
            wgu, wd = gen("experts", lambda: WL.gen_experts(w, self.local, gen_threads))
            self.w_gu, self.w_d = wgu.to(self.dev), wd.to(self.dev)
            sgu, sd = gen("shared", lambda: WL.gen_shared_all(w))
            self.sw_gu = None if sgu is None else sgu.to(self.dev)
            self.sw_d = None if sd is None else sd.to(self.dev)
            can_pack = w.dtype == "bf16" and w.I % 128 == 0 and w.H % 256 == 0
            if pack is None:
                pack = can_pack
            if pack and not can_pack:
                raise ValueError("packed weights need bf16, I % 128 == 0 and H % 256 == 0")
            self.packed = bool(pack)
            if self.packed and not inputs_packed:
                # one-time weight preparation (as at model load): the same values, permuted
                self.w_gu = moe.moe_pack_weights(self.w_gu, 2)
                self.w_d = moe.moe_pack_weights(self.w_d, 1)
                if self.sw_gu is not None:
                    self.sw_gu = moe.moe_pack_weights(self.sw_gu, 2)
                    self.sw_d = moe.moe_pack_weights(self.sw_d, 1)
                torch.cuda.synchronize()
        else:
            self.w_gu = self.w_d = self.sw_gu = self.sw_d = None
            self.packed = False

        # outputs and workspaces
        self.topk_idx = torch.empty((N, k), dtype=torch.int32, device=self.dev)
        self.topk_w = torch.empty((N, k), dtype=torch.float32, device=self.dev)
        self.layout = moe.Layout(N, E, k, W, H, device=self.dev)
        if w.dst_rank < 0:
            cap = N * kw if w.dedup else N * k
        else:
            cap = N if w.dedup else N * min(k, self.e_loc)
        self.rows = torch.empty((cap, H), dtype=dt, device=self.dev)
        self.max_rows = N * k if w.dst_rank < 0 else N * min(k, self.e_loc)
        if self.swiglu:
            self.h = torch.empty((self.max_rows, w.I), dtype=dt, device=self.dev)
            # expert outputs of every rank in row order (rank dst_rank's rows come from the FFN)
            self.y = torch.empty((N * k, H), dtype=dt, device=self.dev)
            S = w.n_shared
            self.sh_h = torch.empty((S, N, w.I), dtype=dt, device=self.dev) if S else None
            self.sh_y = torch.empty((S, N, H), dtype=dt, device=self.dev) if S else None
        else:
            self.h = self.sh_h = self.sh_y = None
            self.y = self.rows
        t0, t1 = w.owned
        self.out = torch.empty((t1 - t0, H), dtype=dt, device=self.dev)
        self.partial = torch.empty((N * kw, H), dtype=dt, device=self.dev) if w.dedup else None
        self._standins_placed = w.dst_rank < 0

    # --------------------------------------------------------------------------------------
    def route(self):
        """Top-k from the stored logits; also writes the layout's count rows, so dispatch()
        skips its count step."""
        moe.moe_route(self.logits, self.bias, self.w.k, self.w.gate, self.topk_idx, self.topk_w,
                      counts=(self.layout, self.placement))
        self._counted = True

    def gate_route(self):
        """Route from x: router linear layer on the device (logits written to self.gate_logits),
        then the same top-k selection."""
        if getattr(self, "w_router", None) is None:
            self.w_router = torch.from_numpy(WL.gen_router(self.w)).to(self.dev)
            self.gate_logits = torch.empty((self.w.N, self.w.E), dtype=torch.float32,
                                           device=self.dev)
            # the router weights are split into bf16 high part and remainder once, at set-up
            self.gate_ws = moe.moe_gate_prepare(self.w_router)
        moe.moe_gate_route(self.x, self.w_router, self.bias, self.w.k, self.w.gate,
                           self.gate_logits, self.topk_idx, self.topk_w, workspace=self.gate_ws,
                           counts=(self.layout, self.placement), prepared=True)
        self._counted = True

    def dispatch(self):
        """Layout and permute of the current routing (the count rows come from the route that
        produced it; without one, the layout counts itself)."""
        moe.moe_dispatch_layout(self.layout, self.topk_idx, self.placement, self.x,
                                dedup=self.w.dedup, dst_rank=self.w.dst_rank, rows_out=self.rows,
                                counts_ready=getattr(self, "_counted", False))

    def ffn(self, phases=3, routed=True, shared=True):
        """The expert FFN: routed groups and shared experts in the same launches, or either part
        alone (routed=False: the shared experts only, which need no routing)."""
        if not self.swiglu:
            return
        w, L = self.w, self.layout
        has_shared = shared and self.sw_gu is not None
        if not routed:
            if has_shared:
                moe.moe_expert_ffn(None, None, 0, None, None, None, None, 0, shared_x=self.x,
                                   shared_w_gate_up=self.sw_gu, shared_w_down=self.sw_d,
                                   shared_h=self.sh_h, shared_y=self.sh_y, phases=phases,
                                   weights_packed=self.packed)
            return
        r = max(w.dst_rank, 0)
        G = len(self.local)
        gather = gbase = None
        if w.dedup:
            gather = L.ptr("expand_src")
            if w.dst_rank >= 0:
                gbase = L.ptr("pair_offsets", r)
        moe.moe_expert_ffn(self.rows, L.ptr("group_offsets", r * self.e_loc if w.dst_rank >= 0
                                            else 0), G, self.w_gu, self.w_d, self.h, self.y,
                           self.max_rows, row_gather=gather, gather_base=gbase,
                           y_absolute=True,
                           shared_x=self.x if has_shared else None,
                           shared_w_gate_up=self.sw_gu if has_shared else None,
                           shared_w_down=self.sw_d if has_shared else None,
                           shared_h=self.sh_h if has_shared else None,
                           shared_y=self.sh_y if has_shared else None, phases=phases,
                           weights_packed=self.packed)

    def combine(self):
        w = self.w
        if not self._standins_placed:
            raise RuntimeError("one rank's share: call place_standins() after the first route "
                               "and dispatch, before the first combine")
        t0, t1 = w.owned
        moe.moe_combine(self.layout, self.y, self.topk_idx, self.topk_w, self.out,
                        expert_rank=self.placement, dedup=w.dedup, t_begin=t0, t_end=t1,
                        shared=self.sh_y, partial=self.partial,
                        y_is_pair_rows=w.dedup and not self.swiglu, dst_rank=w.dst_rank)

    def step(self, fused_gate=False, overlap_shared=False):
        """One pass of the whole hot path. overlap_shared: the shared experts, which need no
        routing, run on a second stream while route, dispatch and the routed experts run on the
        current one; the combine waits for both."""
        if overlap_shared and self.swiglu and self.sw_gu is not None:
            main = torch.cuda.current_stream()
            if getattr(self, "side", None) is None:
                self.side = torch.cuda.Stream(device=self.dev)
            self.side.wait_stream(main)           # x ready; the last combine read sh_y
            with torch.cuda.stream(self.side):
                self.ffn(routed=False)
            self.gate_route() if fused_gate else self.route()
            self.dispatch()
            self.ffn(shared=False)
            main.wait_stream(self.side)
            self.combine()
            return
        if fused_gate:
            self.gate_route()
        else:
            self.route()
        self.dispatch()
        self.ffn()
        self.combine()

    def capture(self, fused_gate=False, overlap_shared=False):
        """Records one step into a HIP graph (every call of the step is a kernel launch; nothing
        in it allocates, synchronises or sets memory; with overlap_shared the second stream
        forks from and joins the capture stream). Run an eager step first so that one-time
        set-up (occupancy queries, stand-ins) is outside the graph. Returns the graph;
        graph.replay() runs the step on the same buffers."""
        g = torch.cuda.CUDAGraph()
        warm = torch.cuda.Stream()
        warm.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(warm):
            self.step(fused_gate, overlap_shared)   # warm-up on the capture stream
        torch.cuda.current_stream().wait_stream(warm)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            self.step(fused_gate, overlap_shared)
        torch.cuda.synchronize()
        self.graph = g
        return g

    # --------------------------------------------------------------------------------------
    def place_standins(self, standin=None):
        """Writes the other ranks' stand-in rows for the owned tokens into y (set-up, once,
        after a route + dispatch; needs a synchronisation). With dedup, the other ranks send
        weighted partials instead: one combine over every pair row turns the stand-in rows into
        those partials (the step's combine then recomputes only rank dst_rank's own partials)."""
        w = self.w
        if w.dst_rank < 0:
            return
        standin = WL.gen_standin(w) if standin is None else standin
        t0, t1 = w.owned
        torch.cuda.synchronize()
        idx = self.topk_idx[t0:t1].long()
        rank = idx // self.e_loc
        remote = (rank != w.dst_rank).reshape(-1)
        rows = self.layout["row_of_slot"][t0 * w.k:t1 * w.k].long()[remote]
        vals = standin.reshape(-1, w.H).to(self.dev)[remote]
        if w.dedup:
            self.y.zero_()
        self.y.index_copy_(0, rows, vals)
        if w.dedup:
            moe.moe_combine(self.layout, self.y, self.topk_idx, self.topk_w, self.out,
                            expert_rank=self.placement, dedup=True, t_begin=t0, t_end=t1,
                            partial=self.partial, dst_rank=-1)
        torch.cuda.synchronize()
        self._standins_placed = True


class MicrobatchLayer:
    """The layer step over M microbatches of N / M consecutive tokens, pipelined over three
    streams: route and dispatch of microbatch i + 1 run while the expert FFN of microbatch i
    runs, and the combine of microbatch i follows its FFN (blog "Kernel fusion for expert
    parallelism", section "Fusing the layer into one kernel": microbatches pipelined through the
    layer's stages; here each stage is the library's own launches, ordered by events, instead of
    one fused launch). Every microbatch has its own layout and row buffers; the expert and
    shared weights are the full layer's, shared. Each token's output equals the unsplit step's:
    routing, the expert rows and the combine are per token, and a row's GEMM result does not
    depend on the other rows of its tile.

    Workloads that run every rank's share (dst_rank = -1) only; N must split into M
    microbatches of a multiple of W tokens. full: an existing MoELayerRun of the workload whose
    inputs and weights the microbatches take (default: a new one)."""

    def __init__(self, w: WL.Workload, M: int, device="cuda", full=None):
        if w.dst_rank >= 0:
            raise ValueError("microbatches need a workload that runs every rank's share")
        if M < 1 or w.N % M or (w.N // M) % w.W:
            raise ValueError("N must split into M microbatches of a multiple of W tokens")
        self.w, self.M = w, M
        self.full = MoELayerRun(w, device=device) if full is None else full
        f = self.full
        n = w.N // M
        sub = WL.shrink(w, N=n)
        logits = np.asarray(f.host["logits"])
        self.subs = []
        for i in range(M):
            inputs = {"x": f.x[i * n:(i + 1) * n], "logits": logits[i * n:(i + 1) * n],
                      "bias": f.host["bias"]}
            if f.swiglu:
                inputs["experts"] = (f.w_gu, f.w_d)
                inputs["shared"] = (f.sw_gu, f.sw_d)
            self.subs.append(MoELayerRun(sub, device=device, inputs=inputs, pack=f.packed,
                                         inputs_packed=f.packed))
        self.streams = None

    def step(self):
        """One pipelined pass over the M microbatches; the current stream waits for all of it."""
        main = torch.cuda.current_stream()
        if self.streams is None:
            self.streams = [torch.cuda.Stream(device=self.full.dev) for _ in range(3)]
        s_disp, s_ffn, s_comb = self.streams
        for s in self.streams:
            s.wait_stream(main)
        for r in self.subs:
            with torch.cuda.stream(s_disp):
                r.route()
                r.dispatch()
                dispatched = torch.cuda.Event()
                dispatched.record(s_disp)
            with torch.cuda.stream(s_ffn):
                s_ffn.wait_event(dispatched)
                r.ffn()
                done = torch.cuda.Event()
                done.record(s_ffn)
            with torch.cuda.stream(s_comb):
                s_comb.wait_event(done)
                r.combine()
        for s in self.streams:
            main.wait_stream(s)

    def outputs(self) -> torch.Tensor:
        """The layer output [N, H] (microbatch outputs in token order)."""
        return torch.cat([r.out for r in self.subs])


class FusedLayerRun:
    """The layer of a MoELayerRun as one launch (moe_layer_fused, for small batches) on the same
    inputs and weights (plain or packed): route from the stored logits, every rank's share, the
    flat combine."""

    def __init__(self, run: MoELayerRun):
        w = run.w
        if not run.swiglu or w.dst_rank >= 0 or w.dedup:
            raise ValueError("the fused layer runs SwiGLU experts over every rank's share with "
                             "the flat combine")
        self.run = run
        self.out = torch.empty_like(run.out)
        self.topk_idx = torch.empty_like(run.topk_idx)
        self.topk_w = torch.empty_like(run.topk_w)
        self.ws = None

    def step(self):
        r = self.run
        _, _, _, self.ws = moe.moe_layer_fused(
            r.x, r.logits, r.bias, r.w.k, r.w.gate, r.w_gu, r.w_d, r.sw_gu, r.sw_d,
            workspace=self.ws, out=self.out, topk_idx=self.topk_idx, topk_w=self.topk_w,
            weights_packed=r.packed)

    def error(self) -> int:
        return moe.fused_error(self.ws)

