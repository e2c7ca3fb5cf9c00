"""One MoE layer step on one rank, as a sequence of libmoe.so calls.

Buffers are allocated once (static shapes: every rank receives exactly S*K
rows, so nothing here depends on the routing).  ``forward`` and
``backward`` only enqueue C-ABI calls on torch's current stream (and, with
``overlap``, the backward on a second stream joined back into it); every
number is computed by the HIP kernels.

In one stream (``overlap=False``):
Forward (rank r):  plan -> dispatch layout -> prefetch slot rows of both
projections -> permute -> up GEMM -> down GEMM (written into rank r's
slice of the all-ranks expert-output buffer) -> combine.
Backward:          weighted permute of the output gradient (combine's
adjoint for the expert outputs) -> router-weight gradient (combine's
adjoint for the weights) -> down DGRAD -> down WGRAD -> up DGRAD (into rank
r's slice of the all-ranks input-gradient buffer) -> up WGRAD -> un-permute
reduce of the input gradients to the tokens (dispatch's adjoint) -> fold the
replica rows of both weight gradients into their home experts.
With ``plan_noalloc=True`` the plan runs on the library's static scratch
(moe_plan_noalloc) instead of the workspace.
With ``fused_gather=True`` (identity activation) there is no permute and no
xp buffer: the up projection's FWD and WGRAD read their row operand straight
from the token rows through src_flat (moe_group_gemm_gather), the permute
fused into the expert GEMM.
With ``overlap=True`` the backward puts the kernels whose results no later
kernel of the step reads on a second stream, each under a GEMM of the
four-wave form (one workgroup per CU that leaves room on every CU for a row
kernel's waves): the router-weight gradient beside the down DGRAD, and both
folds beside the up DGRAD, which then comes after the up WGRAD.  Events order
them after what they read; the main stream waits for the second one before
the step ends.  The default (``overlap=None``) turns it on for steps with
S*K*H*H' >= kOverlapMinWork, where the GEMMs are long enough to hide the
kernels beside them.
The activation between the projections is the identity, or, with
``activation="swiglu"``, the gated linear unit: the up projection then has
2H' columns holding (gate, up) pairs, its GEMM writes both the pre-activation
h and z = silu(gate) * up, and the backward turns dz into dh with the gated
unit's derivative before the up projection's DGRAD and WGRAD.
"""
from dataclasses import dataclass

import torch

from . import (GEMM_DGRAD, GEMM_FWD, GEMM_WGRAD, dims as _mk_dims, dispatch_layout_workspace_bytes,
               group_gemm_workspace_bytes, moe_combine, moe_combine_weight_grad,
               moe_dispatch_layout, moe_group_gemm, moe_group_gemm_gather, moe_group_gemm_swiglu,
               moe_permute, moe_plan, moe_plan_noalloc,
               moe_prefetch, moe_replica_grad_fold, moe_swiglu_backward, moe_unpermute_reduce,
               plan_words, plan_workspace_bytes)


# S*K*H*H' from which the backward uses its second stream by default (the R32 S4096 K8 H7168
# H'2048 step has 4.8e11; its DGRADs take ~0.8 ms each)
kOverlapMinWork = 1e11


@dataclass
class Shape:
    R: int
    S: int
    K: int
    E: int
    B: int
    H: int
    Hp: int

    @property
    def SK(self):
        return self.S * self.K

    @property
    def G(self):
        return self.E + self.B


class LayerStep:
    def __init__(self, shape: Shape, rank: int = 0, dtype=torch.bfloat16, device="cuda",
                 backward: bool = True, activation: str = "identity", fused_gather: bool = False,
                 plan_noalloc: bool = False, overlap=None):
        s = shape
        if activation not in ("identity", "swiglu"):
            raise ValueError(f"activation {activation!r}")
        if fused_gather and (activation != "identity" or dtype != torch.bfloat16):
            raise ValueError("the gathered (permute-fused) up projection is bf16, identity only")
        self.fused_gather = fused_gather
        # plan with the library's static scratch (moe_plan_noalloc) instead of the workspace
        self.plan_noalloc = plan_noalloc
        self.s, self.rank, self.dtype, self.device = s, rank, dtype, device
        self.activation = activation
        # gated: the up projection has 2H' columns, (gate, up) pairs interleaved
        self.up_cols = 2 * s.Hp if activation == "swiglu" else s.Hp
        self.d = _mk_dims(s.R, s.S, s.K, s.E, s.B)
        i32 = dict(dtype=torch.int32, device=device)
        f32 = dict(dtype=torch.float32, device=device)
        act = dict(dtype=dtype, device=device)
        self.topk_idx = torch.zeros((s.R, s.S, s.K), **i32)
        self.topk_w = torch.zeros((s.R, s.S, s.K), **f32)
        self.counts = torch.zeros((s.R, s.E), **i32)
        self.plan = torch.zeros(plan_words(self.d), **i32)
        self.status = torch.zeros(1, **i32)
        ws = max(plan_workspace_bytes(self.d), dispatch_layout_workspace_bytes(self.d))
        self.ws = torch.zeros(ws, dtype=torch.uint8, device=device)
        # the FWD and DGRAD GEMMs' scratch (split of their last round of tiles); the calls
        # run one after another on one stream, so they share it
        self.gemm_ws = torch.empty(group_gemm_workspace_bytes(GEMM_FWD), dtype=torch.uint8,
                                   device=device) if dtype == torch.bfloat16 else None
        self.cu = torch.zeros(s.G + 1, **i32)
        self.dest = torch.zeros(s.R * s.SK, **i32)
        self.src = torch.zeros(s.SK, **i32)
        self.x_all = torch.zeros((s.R * s.S, s.H), **act)
        self.w_up = torch.zeros((s.G, s.H, self.up_cols), **act)
        self.w_down = torch.zeros((s.G, s.Hp, s.H), **act)
        # the permuted token rows (not needed when the up projection gathers them itself)
        self.xp = None if fused_gather else torch.zeros((s.SK, s.H), **act)
        self.z = torch.zeros((s.SK, s.Hp), **act)
        # gated: the pre-activation, kept for the backward
        self.hpre = torch.zeros((s.SK, self.up_cols), **act) if activation == "swiglu" else None
        self.y_all = torch.zeros((s.R * s.SK, s.H), **act)
        self.out = torch.zeros((s.S, s.H), **act)
        self.backward_enabled = backward
        # the backward's side stream (default priority) and its fork/join events; by default
        # only where the GEMMs are long enough for the kernels beside them to gain more than
        # the cross-stream waits cost (~tens of microseconds on short steps)
        if overlap is None:
            overlap = s.S * s.K * s.H * s.Hp >= kOverlapMinWork
        self.overlap = bool(overlap)
        self.side = torch.cuda.Stream(device=device)
        self.ev_fork, self.ev_wgrad, self.ev_join = (torch.cuda.Event() for _ in range(3))
        if backward:
            self.dout_all = torch.zeros((s.R * s.S, s.H), **act)
            self.dy = torch.zeros((s.SK, s.H), **act)
            self.dz = torch.zeros((s.SK, s.Hp), **act)
            self.dh = torch.zeros((s.SK, self.up_cols), **act) if activation == "swiglu" else None
            # every rank's input-gradient rows in the layout's order; this rank's DGRAD writes
            # its slice, the other slices stand in for the peers' (the un-permute reduce reads
            # a token's K copies wherever they were processed)
            self.dxp_all = torch.zeros((s.R * s.SK, s.H), **act)
            self.dx = torch.zeros((s.S, s.H), **act)
            self.dtopk_w = torch.zeros(s.SK, **f32)
            self.dw_up = torch.zeros((s.G, s.H, self.up_cols), **f32)
            self.dw_down = torch.zeros((s.G, s.Hp, s.H), **f32)

    @property
    def dxp(self):
        """This rank's slice of the input-gradient buffer (the up projection's DGRAD writes here)."""
        r, SK = self.rank, self.s.SK
        return self.dxp_all[r * SK:(r + 1) * SK]

    @property
    def y(self):
        """This rank's slice of the expert-output buffer (the down GEMM writes here)."""
        r, SK = self.rank, self.s.SK
        return self.y_all[r * SK:(r + 1) * SK]

    @staticmethod
    def _call(timer, name, fn, *args):
        if timer is None:
            fn(*args)
        else:
            timer(name, fn, *args)

    def forward(self, timer=None):
        s, r, c = self.s, self.rank, self._call
        if self.plan_noalloc:
            c(timer, "plan", moe_plan_noalloc, self.d, self.topk_idx, self.counts, self.plan,
              self.status)
        else:
            c(timer, "plan", moe_plan, self.d, self.topk_idx, self.counts, self.plan,
              self.status, self.ws)
        c(timer, "dispatch_layout", moe_dispatch_layout, self.d, r, self.topk_idx, self.plan,
          self.cu, self.dest, self.src, self.ws)
        c(timer, "prefetch", moe_prefetch, self.d, r, self.plan, self.w_up)
        c(timer, "prefetch", moe_prefetch, self.d, r, self.plan, self.w_down)
        if self.fused_gather:   # up projection reading the token rows through src_flat
            c(timer, "gemm_fwd_gather", moe_group_gemm_gather, GEMM_FWD, self.x_all, self.src,
              s.K, self.w_up, self.cu, self.z, s.H, s.Hp, self.gemm_ws)
        else:
            c(timer, "permute", moe_permute, self.d, self.x_all, self.src, self.xp)
            if self.activation == "swiglu":
                c(timer, "gemm_fwd_swiglu", moe_group_gemm_swiglu, self.xp, self.w_up, self.cu,
                  self.z, self.hpre, s.H, self.up_cols, self.gemm_ws)
            else:
                c(timer, "gemm_fwd", moe_group_gemm, GEMM_FWD, self.xp, self.w_up, self.cu, self.z,
                  s.H, s.Hp, self.gemm_ws)
        c(timer, "gemm_fwd", moe_group_gemm, GEMM_FWD, self.z, self.w_down, self.cu, self.y, s.Hp,
          s.H, self.gemm_ws)
        c(timer, "combine", moe_combine, self.d, r, self.y_all, self.dest,
          self.topk_w.view(-1), self.out)

    def backward(self, timer=None):
        s, r, c = self.s, self.rank, self._call
        c(timer, "permute_weighted", moe_permute, self.d, self.dout_all, self.src, self.dy,
          self.topk_w.view(-1))
        cwgrad = (timer, "combine_wgrad", moe_combine_weight_grad, self.d, r, self.y_all,
                  self.dest, self.dout_all[r * s.S:(r + 1) * s.S], self.dtopk_w)
        if self.overlap:
            main = torch.cuda.current_stream()
            self.ev_fork.record(main)
        else:
            c(*cwgrad)
        c(timer, "gemm_dgrad", moe_group_gemm, GEMM_DGRAD, self.dy, self.w_down, self.cu, self.dz,
          s.Hp, s.H, self.gemm_ws)
        if self.overlap:  # beside the down DGRAD: it reads only forward results and dout
            self.side.wait_event(self.ev_fork)
            with torch.cuda.stream(self.side):
                c(*cwgrad)
        c(timer, "gemm_wgrad", moe_group_gemm, GEMM_WGRAD, self.z, self.dy, self.cu, self.dw_down,
          s.Hp, s.H)
        dup = self.dz
        if self.activation == "swiglu":
            c(timer, "swiglu_bwd", moe_swiglu_backward, self.hpre, self.dz, self.dh)
            dup = self.dh
        up_dgrad = (timer, "gemm_dgrad", moe_group_gemm, GEMM_DGRAD, dup, self.w_up, self.cu,
                    self.dxp, s.H, self.up_cols, self.gemm_ws)
        if not self.overlap:
            c(*up_dgrad)
        if self.fused_gather:
            c(timer, "gemm_wgrad_gather", moe_group_gemm_gather, GEMM_WGRAD, self.x_all, self.src,
              s.K, dup, self.cu, self.dw_up, s.H, self.up_cols)
        else:
            c(timer, "gemm_wgrad", moe_group_gemm, GEMM_WGRAD, self.xp, dup, self.cu, self.dw_up,
              s.H, self.up_cols)
        folds = ((timer, "fold", moe_replica_grad_fold, self.d, r, self.plan, self.dw_up),
                 (timer, "fold", moe_replica_grad_fold, self.d, r, self.plan, self.dw_down))
        if self.overlap:  # both folds beside the up DGRAD, after both WGRADs
            self.ev_wgrad.record(main)
            c(*up_dgrad)
            self.side.wait_event(self.ev_wgrad)
            with torch.cuda.stream(self.side):
                for f in folds:
                    c(*f)
            self.ev_join.record(self.side)
        c(timer, "unpermute_reduce", moe_unpermute_reduce, self.d, r, self.dxp_all, self.dest,
          self.dx)
        if self.overlap:
            main.wait_event(self.ev_join)
        else:
            for f in folds:
                c(*f)

    def step(self, timer=None):
        self.forward(timer)
        if self.backward_enabled:
            self.backward(timer)
