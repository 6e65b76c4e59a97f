"""One training step of the tensor-parallel MLP sublayer on one GPU.

The S shards of the FFN axis are run one after the other on the same device.
Each shard's work is exactly one tensor-parallel rank's share; the two
all-reduces of the method become tp_partial_sum at the same two points
("Split the contraction" and "Put the other collective in backward",
"Megatron tensor-parallel MLP", synapticradio.com):

  forward   shard s: tp_mlp_forward_ws -> fp32 partial z_s (the down GEMM splits k through the
            step's workspace where it has few tiles)
            out = tp_partial_sum(z_0..z_{S-1}) + x + b_down          (forward boundary)
  backward  shard s: tp_mlp_backward(SHARD, d_out = out) -> dN_s and the shard's weight grads
            tp_mlp_backward(NORM, d_normed_parts = dN_0..dN_{S-1})   (backward boundary: the sum
            of the partials formed inside the RMSNorm backward) -> dx, d_norm_w, d_b_down
  update    tp_mlp_sgd_step_multi over every parameter tensor, writing the bf16 weight
            matrices' transposed copies beside them (the backward's d_act and d_normed
            GEMMs read those, so both run with K-contiguous operands), or
            tp_mlp_clip_grad_norm + tp_mlp_adamw_step_multi (copies re-formed after it)

A global batch can be run as microbatches ("Megatron-LM walkthrough", Part IV,
Stage 4): contiguous token slices, each run forward and backward on row views
of the same buffers, the weight gradients accumulated in fp32
(TP_MLP_ACCUMULATE_GRADS) before one optimiser step (Stage 8).

Work that every rank repeats on replicated data (the RMSNorm forward, the
RMSNorm backward, the update of norm_w and b_down) is done once here: its
result is the same on every rank.  With S = 1 there is nothing to sum: the
down projection writes x + z + b_down directly and dN_0 is dN.

The ablations of "Remove each collective" are modes of the same driver:
"missing_forward_reduce" gives each shard its own out_s = x + z_s + b_down
(its own loss and backward; the backward sum is kept), and
"missing_backward_reduce" feeds each shard's own dN_s into the RMSNorm
backward.  Every arithmetic step runs in libtpmlp's kernels; this module only
allocates device memory (through PyTorch) and sequences the C calls.
"""

from __future__ import annotations

from typing import Dict, List, Optional

import torch

from . import _lib as L

MODES = ("equivalence", "missing_forward_reduce", "missing_backward_reduce")


def _torch_dtype(name: str):
    return {"bf16": torch.bfloat16, "fp32": torch.float32}[name]


def _wgrad_ksplit(M: int, N: int, K: int) -> int:
    """The k-slice count the library gives a bf16 weight-gradient GEMM of this
    shape (a function of the shape: fewer than 192 tiles of 256 x 256 take the
    most slices, at most 8, that keep one round of 256 CUs and 1024 of k each)."""
    tiles = -(-M // 256) * -(-N // 256)
    if tiles >= 192:
        return 1
    ks = 1
    while ks < 8 and tiles * (ks + 1) <= 256 and K // (ks + 1) >= 1024:
        ks += 1
    return ks


def microbatch_bounds(tokens: int, microbatches: int) -> List[tuple]:
    """Contiguous token slices [lo, hi): the first tokens % microbatches
    slices hold one token more than the rest."""
    if microbatches < 1:
        raise ValueError("microbatches must be >= 1")
    base, extra = divmod(tokens, microbatches)
    out, lo = [], 0
    for i in range(microbatches):
        hi = lo + base + (1 if i < extra else 0)
        out.append((lo, hi))
        lo = hi
    return out


def sequence_slices(tokens: int, ranks: int) -> List[tuple]:
    """Token rows [lo, hi) of each sequence-parallel rank (the sequence axis
    is outermost in [T, H], so a rank's slice is a contiguous row block)."""
    return microbatch_bounds(tokens, ranks)


class ShardedStep:
    """Device buffers and the call sequence of one step of a workload.

    ``w`` is a ``synth.Workload`` (tokens, hidden, ffn_full, shards, act,
    dtype, eps, lr, master, n_run); ``tensors`` the dense CPU tensors of
    ``synth.draw``.  With ``out_of_place_sgd`` the update writes new
    parameter buffers and leaves the inputs unchanged, so repeated steps do
    identical work (benchmarking); otherwise parameters update in place.
    With ``fused_sgd`` (bf16) a step's SGD update of every shard's w_in and
    w_down is taken inside the SHARD backward, in their weight-gradient GEMMs
    (tp_mlp_fused_sgd): those gradients are then never written, and the
    separate update covers the remaining parameters.  The new parameters are
    the same bits as without it.
    """

    def __init__(self, w, tensors: Dict[str, torch.Tensor], device="cuda", out_of_place_sgd: bool = False,
                 stream: Optional[torch.cuda.Stream] = None, fused_sgd: bool = False):
        if fused_sgd and w.dtype != "bf16":
            raise ValueError("the fused update is bf16 only")
        self.fused_sgd = fused_sgd
        self._fused_names: set = set()
        self.w = w
        self.dev = torch.device(device)
        self.stream = stream
        self.dt = _torch_dtype(w.dtype)
        self.cdt = L.BF16 if w.dtype == "bf16" else L.F32
        self.act = L.ACT_SWIGLU if w.act == "swiglu" else L.ACT_GELU
        self.swiglu = w.act == "swiglu"
        T, H, F = w.tokens, w.hidden, w.ffn_local
        if w.ffn_full % w.shards:
            raise ValueError("ffn_full must be divisible by shards")
        self.T, self.H, self.F = T, H, F
        self.fuse = w.shards == 1
        self.oop = out_of_place_sgd
        dev, dt, f32 = self.dev, self.dt, torch.float32
        up = lambda t: None if t is None else t.to(dev).contiguous()
        emp = lambda shape, d=dt: torch.empty(shape, dtype=d, device=dev)

        self.x = up(tensors["x"])
        self.norm_w = up(tensors["norm_w"])
        self.b_down = up(tensors["b_down"])
        P = 2 * F if self.swiglu else F
        self.shards: List[dict] = []
        for s in range(w.n_run):
            lo, hi = s * F, (s + 1) * F
            sh = {}
            sh["w_in"] = up(tensors["w_in"][:, lo:hi, :] if self.swiglu else tensors["w_in"][lo:hi, :])
            sh["w_down"] = up(tensors["w_down"][:, lo:hi])
            sh["b_in"] = None if self.swiglu else up(tensors["b_in"][lo:hi])
            sh["pre"] = emp((T, P))
            sh["act"] = emp((T, F))
            sh["z"] = None if self.fuse else emp((T, H), f32)
            sh["d_pre"] = emp((T, P))
            sh["d_w_in"] = emp(sh["w_in"].shape, f32)
            sh["d_b_in"] = None if self.swiglu else emp((F,), f32)
            sh["d_w_down"] = emp((H, F), f32)
            sh["dN_part"] = emp((T, H), f32)
            # bf16: each weight matrix is also kept transposed -- w_down as [F, H] for the
            # d_act GEMM, w_in as [H, P] for the d_normed GEMM -- formed once here and then
            # written by every SGD update beside the weight
            sh["w_down_t"] = sh["w_in_t"] = None
            if self.cdt == L.BF16:
                sh["w_down_t"] = emp((F, H))
                L.tp_mlp_transpose_bf16(sh["w_down"], sh["w_down_t"], H, F, stream=stream)
                sh["w_in_t"] = emp((H, P))
                L.tp_mlp_transpose_bf16(sh["w_in"], sh["w_in_t"], P, H, stream=stream)
            self.shards.append(sh)
        self.normed = emp((T, H))
        self.rstd = emp((T,), f32)
        # The fused update's w_in weight-gradient GEMM on K-contiguous operands: N and d_pre transposed
        # ([H, T] once per step, [P, T] per shard in one shared buffer), when the library takes that path
        # (no masters, T a multiple of 8, a k range the GEMM does not split).
        self.normed_t = self.d_pre_t = None
        if fused_sgd and not w.master and T % 8 == 0 and T > 0 and _wgrad_ksplit(P, H, T) == 1:
            self.normed_t = emp((H, T))
            self.d_pre_t = emp((P, T))
        self.out = emp((T, H))
        self.dN = self.shards[0]["dN_part"] if self.fuse else emp((T, H), f32)
        self.dx = emp((T, H))
        self.d_norm_w = emp((H,), f32)
        self.d_b_down = emp((H,), f32)

        # fp32 master copies of every parameter (exact upcasts of the bf16 values)
        self.masters = None
        if w.master:
            self.masters = {}
            for name, t in self._param_list():
                self.masters[name] = t.float().clone()
        # targets of the update
        self.new = {}
        self.new_masters = {}
        # the transposed copies written with the update: name -> (target, rows, cols of the weight)
        self.new_t = {}
        for s, sh in enumerate(self.shards):
            for key, rows, cols in (("w_down", H, F), ("w_in", P, H)):
                tt = sh[key + "_t"]
                if tt is not None:
                    self.new_t[f"{key}.{s}"] = (torch.empty_like(tt) if self.oop else tt, rows, cols)
        for name, t in self._param_list():
            self.new[name] = torch.empty_like(t) if self.oop else t
            if self.masters is not None:
                self.new_masters[name] = torch.empty_like(self.masters[name]) if self.oop else self.masters[name]

        # one workspace for the forward's k-split slices and the backward's scratch (never in use together)
        ws = max(L.tp_mlp_workspace_bytes(self._desc(), L.BWD_NORM),
                 L.tp_mlp_workspace_bytes(self._desc(), L.BWD_SHARD),
                 L.tp_mlp_forward_workspace_bytes(self._desc(L.FUSE_EPILOGUE if self.fuse else 0)), 16)
        self.workspace = torch.empty(ws, dtype=torch.uint8, device=dev)
        # AdamW state, allocated by the first adamw() call
        self.adam_m: Optional[Dict[str, torch.Tensor]] = None
        self.adam_v: Optional[Dict[str, torch.Tensor]] = None
        self.adam_steps = 0
        # per-shard outputs of the ablation modes, allocated on first use
        self._abl: Dict[str, list] = {}
        # the last backward summed dN inside the RMSNorm backward (dN's buffer not written)
        self._dN_streamed = False

    # ------------------------------------------------------------ helpers
    def _desc(self, flags: int = 0, tokens: Optional[int] = None) -> L.tp_mlp_desc:
        w = self.w
        return L.make_desc(self.T if tokens is None else tokens, self.H, self.F, self.act, self.cdt, w.eps, flags)

    def _param_list(self):
        out = [("norm_w", self.norm_w), ("b_down", self.b_down)]
        for s, sh in enumerate(self.shards):
            out.append((f"w_in.{s}", sh["w_in"]))
            out.append((f"w_down.{s}", sh["w_down"]))
            if sh["b_in"] is not None:
                out.append((f"b_in.{s}", sh["b_in"]))
        return out

    def _grad_of(self, name: str) -> torch.Tensor:
        if name == "norm_w":
            return self.d_norm_w
        if name == "b_down":
            return self.d_b_down
        key, s = name.split(".")
        return self.shards[int(s)]["d_" + key]

    def _abl_bufs(self, name, shape, dtype):
        if name not in self._abl:
            self._abl[name] = [torch.empty(shape, dtype=dtype, device=self.dev) for _ in self.shards]
        return self._abl[name]

    # -------------------------------------------------------------- phases
    def forward(self, mode: str = "equivalence", rows: Optional[slice] = None) -> None:
        """Forward of every shard on token rows ``rows`` (default: all)."""
        r = rows if rows is not None else slice(0, self.T)
        T, H = r.stop - r.start, self.H
        st = self.stream
        for s, sh in enumerate(self.shards):
            flags = (L.NORMED_READY if s > 0 else 0) | (L.FUSE_EPILOGUE if self.fuse else 0)
            L.tp_mlp_forward_ws(self._desc(flags, T), self.x[r], self.norm_w, sh["w_in"], sh["b_in"], sh["w_down"],
                                self.normed[r], self.rstd[r], sh["pre"][r], sh["act"][r],
                                self.out[r] if self.fuse else sh["z"][r], self.b_down, workspace=self.workspace,
                                stream=st)
        if self.fuse:
            return
        if rows is not None:
            if mode != "equivalence":
                raise ValueError("microbatches run in equivalence mode only")
            L.tp_partial_sum([sh["z"][r] for sh in self.shards], T, H, self.x[r], self.b_down, self.cdt, self.out[r],
                             self.cdt, stream=st)
            return
        if mode == "missing_forward_reduce":
            outs = self._abl_bufs("out", (T, H), self.dt)
            for sh, o in zip(self.shards, outs):
                L.tp_partial_sum([sh["z"]], T, H, self.x, self.b_down, self.cdt, o, self.cdt, stream=st)
        else:
            L.tp_partial_sum([sh["z"] for sh in self.shards], T, H, self.x, self.b_down, self.cdt, self.out,
                             self.cdt, stream=st)

    def _fused_update(self, s: int, transposed: bool = True) -> dict:
        """The tp_mlp_fused_sgd fields of shard s: its w_in and w_down updated
        into the same targets (and transposed copies, masters) as sgd();
        without ``transposed`` the transposed copies are not written."""
        f = {"lr": self.w.lr}
        for key in ("w_in", "w_down"):
            name = f"{key}.{s}"
            f[key + "_out"] = self.new[name]
            f[key + "_t_out"] = self.new_t[name][0] if (transposed and name in self.new_t) else None
            if self.masters is not None:
                f[key + "_master"] = self.masters[name]
                f[key + "_master_out"] = self.new_masters[name]
            self._fused_names.add(name)
        return f

    def _shard_backward(self, sh, d_out, r: slice = slice(None), flags: int = 0, fused: Optional[dict] = None) -> None:
        T = self.T if r.start is None else r.stop - r.start
        grads = {} if fused else dict(d_w_in=sh["d_w_in"], d_w_down=sh["d_w_down"])
        if fused and self.d_pre_t is not None:
            grads.update(normed_t=self.normed_t, d_pre_t=self.d_pre_t)
        L.tp_mlp_backward(self._desc(flags, T), L.BWD_SHARD, stream=self.stream, normed=self.normed[r],
                          pre_act=sh["pre"][r], act=sh["act"][r], w_in=sh["w_in"], w_down=sh["w_down"],
                          d_out=d_out, d_pre=sh["d_pre"][r], d_b_in=sh["d_b_in"],
                          d_normed_part=sh["dN_part"][r], w_down_t=sh["w_down_t"],
                          w_in_t=sh["w_in_t"], workspace=self.workspace, fused_sgd=fused, **grads)

    def _norm_backward(self, dN, d_out, dx, d_norm_w, d_b_down, r: slice = slice(None), flags: int = 0,
                       parts=None) -> None:
        """The NORM phase on the summed dN, or with ``parts`` (the shards'
        partials of dN) summed by the RMSNorm backward as it reads them."""
        T = self.T if r.start is None else r.stop - r.start
        kw = dict(d_normed_parts=parts) if parts else dict(d_normed=dN)
        L.tp_mlp_backward(self._desc(flags, T), L.BWD_NORM, stream=self.stream, x=self.x[r], rstd=self.rstd[r],
                          norm_w=self.norm_w, d_out=d_out, d_x=dx, d_norm_w=d_norm_w, d_b_down=d_b_down,
                          workspace=self.workspace, **kw)

    def materialize_dN(self) -> None:
        """Write the summed dN into its buffer when the step streamed the
        shards' partials into the RMSNorm backward instead (tp_partial_sum:
        the same sum, in the same order, so the same bits the backward used)."""
        if self._dN_streamed and not self.fuse:
            L.tp_partial_sum([sh["dN_part"] for sh in self.shards], self.T, self.H, None, None, L.F32, self.dN, L.F32,
                             stream=self.stream)
        self._dN_streamed = False

    def backward_rows(self, rows: slice, accumulate: bool) -> None:
        """Backward of one microbatch (token rows ``rows``, equivalence mode);
        with ``accumulate`` the weight gradients are added to the buffers."""
        r, T, H = rows, rows.stop - rows.start, self.H
        flags = L.ACCUMULATE_GRADS if accumulate else 0
        self._fused_names = set()
        for sh in self.shards:
            self._shard_backward(sh, self.out[r], r, flags)
        # the backward boundary: the shards' partials summed inside the RMSNorm backward
        parts = None if self.fuse else [sh["dN_part"][r] for sh in self.shards]
        self._norm_backward(self.dN[r], self.out[r], self.dx[r], self.d_norm_w, self.d_b_down, r, flags, parts=parts)
        self._dN_streamed = not self.fuse

    def backward(self, mode: str = "equivalence", fused_update: bool = False) -> None:
        """The backward of every shard, then the NORM phase.  With
        ``fused_update`` (equivalence mode, ``fused_sgd`` steps) the shards'
        w_in and w_down are updated inside the SHARD phase and their
        gradients are not written; sgd() then updates the rest."""
        T, H = self.T, self.H
        fwd_abl = mode == "missing_forward_reduce" and not self.fuse
        outs = self._abl["out"] if fwd_abl else [self.out] * len(self.shards)
        if fused_update and mode != "equivalence":
            raise ValueError("the fused update runs in equivalence mode only")
        self._fused_names = set()
        if fused_update and self.normed_t is not None:
            L.tp_mlp_transpose_bf16(self.normed, self.normed_t, T, H, stream=self.stream)
        for s, (sh, o) in enumerate(zip(self.shards, outs)):
            self._shard_backward(sh, o, fused=self._fused_update(s) if fused_update else None)
        if mode == "equivalence" or self.fuse:
            # the backward boundary: the shards' partials summed inside the RMSNorm backward
            parts = None if self.fuse else [sh["dN_part"] for sh in self.shards]
            self._norm_backward(self.dN, self.out, self.dx, self.d_norm_w, self.d_b_down, parts=parts)
            self._dN_streamed = not self.fuse
            return
        if mode != "missing_backward_reduce":
            L.tp_partial_sum([sh["dN_part"] for sh in self.shards], T, H, None, None, L.F32, self.dN, L.F32,
                             stream=self.stream)
        dxs = self._abl_bufs("dx", (T, H), self.dt)
        dws = self._abl_bufs("d_norm_w", (H,), torch.float32)
        dbs = self._abl_bufs("d_b_down", (H,), torch.float32)
        for s, sh in enumerate(self.shards):
            dN = self.dN if fwd_abl else sh["dN_part"]
            self._norm_backward(dN, outs[s], dxs[s], dws[s], dbs[s])

    def sgd(self) -> None:
        """One SGD update of every parameter tensor (one launch), except
        those the last backward already updated (fused_update)."""
        lst = []
        for name, t in self._param_list():
            if name in self._fused_names:
                continue
            g = self._grad_of(name)
            if self.masters is not None:
                e = (t, self.new[name], g, self.masters[name], self.new_masters[name], t.numel())
            else:
                e = (t, self.new[name], g, None, None, t.numel())
            if name in self.new_t:  # the weight's transposed copy, written with it
                e = e + self.new_t[name]
            lst.append(e)
        L.tp_mlp_sgd_step_multi(lst, self.cdt, self.w.lr, stream=self.stream)

    def adamw(self, lr: float, weight_decay: float = 0.0, max_norm: float = 0.0, beta1: float = 0.9,
              beta2: float = 0.999, eps: float = 1e-8) -> None:
        """Global-norm clip coefficient, then one AdamW update of every
        parameter tensor (fp32 moments kept on the device; the step count
        advances by one).  Updates go to the same targets as sgd()."""
        params = self._param_list()
        if self.adam_m is None:
            self.adam_m = {n: torch.zeros(t.shape, dtype=torch.float32, device=self.dev) for n, t in params}
            self.adam_v = {n: torch.zeros(t.shape, dtype=torch.float32, device=self.dev) for n, t in params}
            counts = [t.numel() for _, t in params]
            nbytes = max(L.tp_mlp_clip_grad_norm_workspace_bytes(counts), 16)
            self._norm_ws = torch.empty(nbytes, dtype=torch.uint8, device=self.dev)
            self.grad_norm = torch.zeros(1, dtype=torch.float32, device=self.dev)
            self.clip_coef = torch.ones(1, dtype=torch.float32, device=self.dev)
        grads = [self._grad_of(n) for n, _ in params]
        L.tp_mlp_clip_grad_norm(grads, [g.numel() for g in grads], max_norm, self.grad_norm, self.clip_coef,
                                self._norm_ws, stream=self.stream)
        self.adam_steps += 1
        hp = L.make_adamw_hparams(lr, self.adam_steps, weight_decay, beta1, beta2, eps)
        lst = []
        for (name, t), g in zip(params, grads):
            m, v = self.adam_m[name], self.adam_v[name]
            if self.masters is not None:
                lst.append((None, self.new[name], g, self.masters[name], self.new_masters[name], m, v, t.numel()))
            else:
                lst.append((t, self.new[name], g, None, None, m, v, t.numel()))
        L.tp_mlp_adamw_step_multi(lst, self.cdt, hp, grad_scale=self.clip_coef, stream=self.stream)
        for name, (tt, rows, cols) in self.new_t.items():  # the transposed copies follow the update
            L.tp_mlp_transpose_bf16(self.new[name], tt, rows, cols, stream=self.stream)

    def step(self, mode: str = "equivalence", update: bool = True, microbatches: int = 1) -> None:
        """Forward, backward and (``update``) the SGD step.  With
        ``microbatches`` > 1 the tokens run as that many contiguous slices
        whose weight gradients accumulate (equivalence mode only)."""
        if microbatches > 1:
            if mode != "equivalence":
                raise ValueError("microbatches run in equivalence mode only")
            for i, (lo, hi) in enumerate(microbatch_bounds(self.T, microbatches)):
                self.forward(mode, slice(lo, hi))
                self.backward_rows(slice(lo, hi), accumulate=i > 0)
        else:
            self.forward(mode)
            self.backward(mode, fused_update=self.fused_sgd and update and mode == "equivalence")
        if update and mode == "equivalence":
            self.sgd()


    # ------------------------------------------------------------- results
    def results(self, mode: str = "equivalence") -> dict:
        """CPU copies of the step's outputs, shard slices re-assembled along
        the FFN axis.  In ablation modes out/dx/d_norm_w/d_b_down are lists
        over shards."""
        self.materialize_dN()
        c = lambda t: t.detach().float().cpu()
        r = {"normed": c(self.normed), "rstd": c(self.rstd)}
        cat_in = (lambda ts: torch.cat(ts, dim=1)) if self.swiglu else (lambda ts: torch.cat(ts, dim=0))
        if self._fused_names:  # the last backward applied these gradients without writing them
            r["d_w_in"] = r["d_w_down"] = None
        else:
            r["d_w_in"] = cat_in([c(sh["d_w_in"]) for sh in self.shards])
            r["d_w_down"] = torch.cat([c(sh["d_w_down"]) for sh in self.shards], dim=1)
        if not self.swiglu:
            r["d_b_in"] = torch.cat([c(sh["d_b_in"]) for sh in self.shards])
        r["act"] = torch.cat([c(sh["act"]) for sh in self.shards], dim=1)
        r["dN_parts"] = [c(sh["dN_part"]) for sh in self.shards]
        if mode == "equivalence" or self.fuse:
            r.update(out=c(self.out), dx=c(self.dx), d_norm_w=c(self.d_norm_w), d_b_down=c(self.d_b_down),
                     dN=c(self.dN))
        else:
            r["out"] = [c(o) for o in self._abl["out"]] if mode == "missing_forward_reduce" else c(self.out)
            r["dx"] = [c(t) for t in self._abl["dx"]]
            r["d_norm_w"] = [c(t) for t in self._abl["d_norm_w"]]
            r["d_b_down"] = [c(t) for t in self._abl["d_b_down"]]
        new = {name: c(self.new[name]) for name, _ in self._param_list()}
        n = len(self.shards)
        r["new_norm_w"], r["new_b_down"] = new["norm_w"], new["b_down"]
        r["new_w_in"] = cat_in([new[f"w_in.{s}"] for s in range(n)])
        r["new_w_down"] = torch.cat([new[f"w_down.{s}"] for s in range(n)], dim=1)
        if not self.swiglu:
            r["new_b_in"] = torch.cat([new[f"b_in.{s}"] for s in range(n)])
        if self.masters is not None:
            nm = {name: c(self.new_masters[name]) for name, _ in self._param_list()}
            r["master_norm_w"], r["master_b_down"] = nm["norm_w"], nm["b_down"]
            r["master_w_in"] = cat_in([nm[f"w_in.{s}"] for s in range(n)])
            r["master_w_down"] = torch.cat([nm[f"w_down.{s}"] for s in range(n)], dim=1)
        return r


class SequenceParallelStep(ShardedStep):
    """The step in the sequence-parallel layout ("Megatron-LM walkthrough",
    Part V, "Deep dive: sequence parallelism"; Part IV, Stages 5 and 7).

    Rank r of the S ranks owns FFN channels as in ShardedStep and, outside
    the tensor-parallel linears, the contiguous token rows slices[r] of the
    sequence:

      forward   rank r: tp_rmsnorm_forward on its rows -> its rows of N
                (the all-gather entering the region: every rank's rows land
                in the one full N buffer the region reads)
                shard s: tp_mlp_forward(NORMED_READY) on all T rows -> z_s
                rank r: tp_partial_sum of rows slices[r] of z_0..z_{S-1}
                + x + b_down -> its rows of out    (the reduce-scatter)
      backward  shard s: tp_mlp_backward(SHARD) with d_out = out on all rows
                (the all-gather of dY) -> dN_s
                rank r: tp_mlp_backward(NORM) on its rows with its rows of
                dN_0..dN_{S-1} as d_normed_parts (the reduce-scatter, summed
                inside the RMSNorm backward) -> its rows of dx and its own
                d_norm_w, d_b_down
                d_norm_w, d_b_down = tp_partial_sum over the ranks (the
                replicated parameters' gradients summed over the group)

    Mode "missing_norm_grad_reduce" leaves out that last sum: each rank keeps
    the gradient of its own rows.  Every rank runs, one after the other."""

    MODES = ("equivalence", "missing_norm_grad_reduce")

    def __init__(self, w, tensors, device="cuda", out_of_place_sgd: bool = False, stream=None,
                 fused_sgd: bool = False):
        super().__init__(w, tensors, device, out_of_place_sgd, stream, fused_sgd=fused_sgd)
        if w.n_run != w.shards:
            raise ValueError("the sequence-parallel step runs every rank")
        S, H = w.shards, self.H
        self.slices = sequence_slices(self.T, S)
        self.rank_d_norm_w = torch.empty((S, H), dtype=torch.float32, device=self.dev)
        self.rank_d_b_down = torch.empty((S, H), dtype=torch.float32, device=self.dev)

    def forward(self, mode: str = "equivalence", rows=None) -> None:
        if rows is not None:
            raise ValueError("the sequence-parallel step takes the whole batch")
        T, H, st = self.T, self.H, self.stream
        for lo, hi in self.slices:
            L.tp_rmsnorm_forward(hi - lo, H, self.cdt, self.w.eps, self.x[lo:hi], self.norm_w, self.normed[lo:hi],
                                 self.rstd[lo:hi], stream=st)
        for sh in self.shards:
            flags = L.NORMED_READY | (L.FUSE_EPILOGUE if self.fuse else 0)
            L.tp_mlp_forward_ws(self._desc(flags), self.x, self.norm_w, sh["w_in"], sh["b_in"], sh["w_down"],
                                self.normed, self.rstd, sh["pre"], sh["act"], self.out if self.fuse else sh["z"],
                                self.b_down, workspace=self.workspace, stream=st)
        if self.fuse:
            return
        for lo, hi in self.slices:
            L.tp_partial_sum([sh["z"][lo:hi] for sh in self.shards], hi - lo, H, self.x[lo:hi], self.b_down, self.cdt,
                             self.out[lo:hi], self.cdt, stream=st)

    def backward(self, mode: str = "equivalence", fused_update: bool = False) -> None:
        if mode not in self.MODES:
            raise ValueError(mode)
        T, H = self.T, self.H
        self._fused_names = set()
        if fused_update and self.normed_t is not None:
            L.tp_mlp_transpose_bf16(self.normed, self.normed_t, T, H, stream=self.stream)
        for s, sh in enumerate(self.shards):
            self._shard_backward(sh, self.out, fused=self._fused_update(s) if fused_update else None)
        for r, (lo, hi) in enumerate(self.slices):
            # the reduce-scatter of dN: each rank's rows of the partials, summed inside its RMSNorm backward
            parts = None if self.fuse else [sh["dN_part"][lo:hi] for sh in self.shards]
            self._norm_backward(self.dN[lo:hi], self.out[lo:hi], self.dx[lo:hi], self.rank_d_norm_w[r],
                                self.rank_d_b_down[r], slice(lo, hi), parts=parts)
        self._dN_streamed = not self.fuse
        if mode == "equivalence":
            S = len(self.slices)
            L.tp_partial_sum([self.rank_d_norm_w[r] for r in range(S)], 1, H, None, None, L.F32, self.d_norm_w, L.F32,
                             stream=self.stream)
            L.tp_partial_sum([self.rank_d_b_down[r] for r in range(S)], 1, H, None, None, L.F32, self.d_b_down,
                             L.F32, stream=self.stream)

    def step(self, mode: str = "equivalence", update: bool = True, microbatches: int = 1) -> None:
        if microbatches != 1:
            raise ValueError("the sequence-parallel step takes the whole batch")
        self.forward(mode)
        self.backward(mode, fused_update=self.fused_sgd and update and mode == "equivalence")
        if update and mode == "equivalence":
            self.sgd()

    def results(self, mode: str = "equivalence") -> dict:
        r = super().results("equivalence")
        if mode == "missing_norm_grad_reduce":
            c = lambda t: t.detach().float().cpu()
            r["d_norm_w"] = [c(t) for t in self.rank_d_norm_w]
            r["d_b_down"] = [c(t) for t in self.rank_d_b_down]
        return r


class Fp8Step(ShardedStep):
    """The step with every GEMM on FP8 codes and per-tensor delayed scaling
    (tp_mlp_forward_fp8 / tp_mlp_backward_fp8; Transformer Engine's FP8 with
    delayed scaling, "Megatron-Core Guide: 5D Distributed Training
    Architecture", feature list item 6).

    One meta per tensor role is shared by all shards, so each role's amax is
    the maximum over the tensor-parallel group; tp_mlp_fp8_update_scales
    renews the scales at the end of every step.  The replicated tensors' codes
    (N and its transpose, dY and its transpose) are cast once, by shard 0's
    calls, like the replicated RMSNorm itself.  The norm backward, the sums and
    the update are those of ShardedStep."""

    ROLES = (("meta_normed", L.FP8_E4M3), ("meta_w_in", L.FP8_E4M3), ("meta_act", L.FP8_E4M3),
             ("meta_w_down", L.FP8_E4M3), ("meta_d_out", L.FP8_E5M2), ("meta_d_pre", L.FP8_E5M2))

    def __init__(self, w, tensors, device="cuda", out_of_place_sgd: bool = False, stream=None,
                 history_len: int = 16, fused_sgd: bool = False):
        if w.dtype != "bf16":
            raise ValueError("the FP8 step takes bf16 tensors")
        super().__init__(w, tensors, device, out_of_place_sgd, stream, fused_sgd=fused_sgd)
        self.normed_t = self.d_pre_t = None  # the FP8 GEMMs read codes (their transposes come with the casts)
        T, H, F = self.T, self.H, self.F
        P, Tp = (2 * F if self.swiglu else F), (T + 15) // 16 * 16
        u8 = lambda shape: torch.empty(shape, dtype=torch.uint8, device=self.dev)
        self.history_len = history_len
        self.metas = {}
        for name, fmt in self.ROLES:
            m = torch.empty(L.fp8_meta_floats(history_len), dtype=torch.float32, device=self.dev)
            L.tp_mlp_fp8_meta_init(m, fmt, history_len, stream=self.stream)
            self.metas[name] = m
        shared = dict(normed_q=u8((T, H)), normed_t=u8((H, Tp)), d_out_q=u8((T, H)), d_out_t=u8((H, Tp)))
        self.codes_shared = shared
        for sh in self.shards:
            codes = dict(w_in_q=u8((P, H)), w_in_t=u8((H, P)), act_q=u8((T, F)), act_t=u8((F, Tp)),
                         w_down_q=u8((H, F)), w_down_t=u8((F, H)), d_pre_q=u8((T, P)), d_pre_t=u8((P, Tp)))
            sh["codes"] = codes
            sh["f8"] = L.make_fp8_args(history_len, **self.metas, **shared, **codes)

    def forward(self, mode: str = "equivalence", rows=None) -> None:
        if rows is not None or mode != "equivalence":
            raise ValueError("the FP8 step runs the whole batch in equivalence mode")
        T, H, st = self.T, self.H, self.stream
        for s, sh in enumerate(self.shards):
            flags = (L.NORMED_READY if s > 0 else 0) | (L.FUSE_EPILOGUE if self.fuse else 0)
            L.tp_mlp_forward_fp8(self._desc(flags), self.x, self.norm_w, sh["w_in"], sh["b_in"], sh["w_down"],
                                 self.normed, self.rstd, sh["pre"], sh["act"], self.out if self.fuse else sh["z"],
                                 self.b_down, sh["f8"], stream=st)
        if not self.fuse:
            L.tp_partial_sum([sh["z"] for sh in self.shards], T, H, self.x, self.b_down, self.cdt, self.out,
                             self.cdt, stream=st)

    def backward(self, mode: str = "equivalence", fused_update: bool = False) -> None:
        """With ``fused_update`` the weight matrices' SGD update is taken in
        their FP8 weight-gradient GEMMs (their bf16 transposed copies, which
        the FP8 GEMMs do not read, are not written)."""
        if mode != "equivalence":
            raise ValueError("the FP8 step runs in equivalence mode")
        T, H = self.T, self.H
        self._fused_names = set()
        for s, sh in enumerate(self.shards):
            flags = L.FP8_SHARED_READY if s > 0 else 0
            grads = dict(fused_sgd=self._fused_update(s, transposed=False)) if fused_update else \
                dict(d_w_in=sh["d_w_in"], d_w_down=sh["d_w_down"])
            L.tp_mlp_backward_fp8(self._desc(flags), L.BWD_SHARD, sh["f8"], stream=self.stream,
                                  normed=self.normed, pre_act=sh["pre"], act=sh["act"], w_in=sh["w_in"],
                                  w_down=sh["w_down"], d_out=self.out, d_pre=sh["d_pre"],
                                  d_b_in=sh["d_b_in"], d_normed_part=sh["dN_part"],
                                  workspace=self.workspace, **grads)
        # the backward boundary: the shards' partials summed inside the RMSNorm backward
        parts = None if self.fuse else [sh["dN_part"] for sh in self.shards]
        self._norm_backward(self.dN, self.out, self.dx, self.d_norm_w, self.d_b_down, parts=parts)
        self._dN_streamed = not self.fuse

    def update_scales(self) -> None:
        L.tp_mlp_fp8_update_scales([self.metas[n] for n, _ in self.ROLES], self.history_len, stream=self.stream)

    def step(self, mode: str = "equivalence", update: bool = True, microbatches: int = 1) -> None:
        if microbatches != 1:
            raise ValueError("the FP8 step takes the whole batch")
        self.forward(mode)
        self.backward(mode, fused_update=self.fused_sgd and update)
        if update:
            self.sgd()
        self.update_scales()

    def meta_state(self) -> dict:
        """{role: (scale, scale_inv, amax, history)} as CPU values."""
        out = {}
        for name, _ in self.ROLES:
            m = self.metas[name].cpu()
            out[name[5:]] = (float(m[0]), float(m[1]), float(m[2]), m[4:].clone())
        return out

    def load_meta_state(self, state: dict) -> None:
        """Restore metas saved by meta_state (or built from another run):
        {role: (scale, scale_inv, amax, history)}."""
        for name, _ in self.ROLES:
            sc, si, am, hist = state[name[5:]]
            m = self.metas[name]
            vals = torch.tensor([sc, si, am, float(m[3])] + [float(h) for h in hist], dtype=torch.float32)
            m.copy_(vals.to(self.dev))



class AttnStep:
    """One training step of the tensor-parallel attention sublayer
    (tp_attn_forward / tp_attn_backward), S shards of complete query/KV head
    groups run one after the other, with the same two sums as the MLP block:

      forward   shard s: tp_attn_forward -> fp32 partial z_s
                out = tp_partial_sum(z_0..z_{S-1}) + x + b_o
      backward  shard s: tp_attn_backward(SHARD, d_out = out) -> dN_s, its weight grads
                tp_attn_backward(NORM, d_normed_parts = dN_0..dN_{S-1}) -> dx, d_norm_w, d_b_o
                (the backward boundary: the partials summed as the RMSNorm backward reads them)
      update    tp_mlp_sgd_step_multi over every parameter tensor

    Shard r owns query heads [r n_q/S, (r+1) n_q/S) and key/value heads
    [r n_kv/S, (r+1) n_kv/S): its rows of the fused w_qkv are those Q, K and V
    heads' rows (in that order) and its columns of w_o those query heads'.
    Modes as ShardedStep ("missing_forward_reduce", "missing_backward_reduce")."""

    MODES = MODES

    def __init__(self, w, tensors: Dict[str, torch.Tensor], device="cuda", out_of_place_sgd: bool = False,
                 stream: Optional[torch.cuda.Stream] = None):
        if w.n_kv % w.shards or w.n_q % w.n_kv:
            raise ValueError("the shards must own complete query/KV head groups")
        self.w, self.dev, self.stream = w, torch.device(device), stream
        self.T, self.H, self.D, S = w.tokens, w.hidden, w.d, w.shards
        self.nq, self.nkv = w.n_q // S, w.n_kv // S
        self.fuse = S == 1
        self.oop = out_of_place_sgd
        dev, bf, f32 = self.dev, torch.bfloat16, torch.float32
        T, H, D, nq, nkv = self.T, self.H, self.D, self.nq, self.nkv
        W, Wo = (nq + 2 * nkv) * D, nq * D
        emp = lambda shape, d=bf: torch.empty(shape, dtype=d, device=dev)
        up = lambda t: t.to(dev).contiguous()
        self.x, self.norm_w, self.b_o = up(tensors["x"]), up(tensors["norm_w"]), up(tensors["b_o"])
        NQ, NKV = w.n_q, w.n_kv
        self.shards: List[dict] = []
        for r in range(S):
            qlo, kvlo = r * nq, r * nkv
            rows = torch.cat([torch.arange(qlo * D, (qlo + nq) * D), NQ * D + torch.arange(kvlo * D, (kvlo + nkv) * D),
                              (NQ + NKV) * D + torch.arange(kvlo * D, (kvlo + nkv) * D)])
            sh = {"w_qkv": up(tensors["w_qkv"][rows]), "w_o": up(tensors["w_o"][:, qlo * D:(qlo + nq) * D]),
                  "qkv": emp((T, W)), "attn_out": emp((T, Wo)), "lse": emp((nq, T), f32),
                  "z": None if self.fuse else emp((T, H), f32), "d_attn_out": emp((T, Wo)), "d_qkv": emp((T, W)),
                  "d_w_qkv": emp((W, H), f32), "d_w_o": emp((H, Wo), f32), "dN_part": emp((T, H), f32),
                  "rows": rows}
            self.shards.append(sh)
        self.normed, self.rstd, self.out = emp((T, H)), emp((T,), f32), emp((T, H))
        self.dN = self.shards[0]["dN_part"] if self.fuse else emp((T, H), f32)
        # the last backward summed dN inside the RMSNorm backward (dN's buffer not written)
        self._dN_streamed = False
        self.dx, self.d_norm_w, self.d_b_o = emp((T, H)), emp((H,), f32), emp((H,), f32)
        self.new = {name: (torch.empty_like(t) if self.oop else t) for name, t in self._param_list()}
        d0 = self._desc()
        ws = max(L.tp_attn_workspace_bytes(d0, L.BWD_SHARD), L.tp_attn_workspace_bytes(d0, L.BWD_NORM),
                 L.tp_attn_forward_workspace_bytes(d0), 16)
        self.workspace = torch.empty(ws, dtype=torch.uint8, device=dev)
        self._abl: Dict[str, list] = {}

    def _desc(self, flags: int = 0) -> L.tp_attn_desc:
        w = self.w
        return L.make_attn_desc(w.batch, w.seq, self.H, self.nq, self.nkv, self.D, w.eps, flags)

    def _param_list(self):
        out = [("norm_w", self.norm_w), ("b_o", self.b_o)]
        for s, sh in enumerate(self.shards):
            out += [(f"w_qkv.{s}", sh["w_qkv"]), (f"w_o.{s}", sh["w_o"])]
        return out

    def _grad_of(self, name: str) -> torch.Tensor:
        if name in ("norm_w", "b_o"):
            return self.d_norm_w if name == "norm_w" else self.d_b_o
        key, s = name.split(".")
        return self.shards[int(s)]["d_" + key]

    def _abl_bufs(self, name, shape, dtype):
        if name not in self._abl:
            self._abl[name] = [torch.empty(shape, dtype=dtype, device=self.dev) for _ in self.shards]
        return self._abl[name]

    def forward(self, mode: str = "equivalence") -> None:
        T, H, st = self.T, self.H, self.stream
        for s, sh in enumerate(self.shards):
            flags = (L.NORMED_READY if s > 0 else 0) | (L.FUSE_EPILOGUE if self.fuse else 0)
            L.tp_attn_forward(self._desc(flags), self.x, self.norm_w, sh["w_qkv"], sh["w_o"], self.normed, self.rstd,
                              sh["qkv"], sh["attn_out"], sh["lse"], self.out if self.fuse else sh["z"], self.b_o,
                              workspace=self.workspace, workspace_bytes=self.workspace.numel(), stream=st)
        if self.fuse:
            return
        if mode == "missing_forward_reduce":
            for sh, o in zip(self.shards, self._abl_bufs("out", (T, H), torch.bfloat16)):
                L.tp_partial_sum([sh["z"]], T, H, self.x, self.b_o, L.BF16, o, L.BF16, stream=st)
        else:
            L.tp_partial_sum([sh["z"] for sh in self.shards], T, H, self.x, self.b_o, L.BF16, self.out, L.BF16,
                             stream=st)

    def _shard_backward(self, sh, d_out) -> None:
        L.tp_attn_backward(self._desc(), L.BWD_SHARD, stream=self.stream, normed=self.normed, qkv=sh["qkv"],
                           attn_out=sh["attn_out"], lse=sh["lse"], w_qkv=sh["w_qkv"], w_o=sh["w_o"], d_out=d_out,
                           d_attn_out=sh["d_attn_out"], d_qkv=sh["d_qkv"], d_w_qkv=sh["d_w_qkv"], d_w_o=sh["d_w_o"],
                           d_normed_part=sh["dN_part"], workspace=self.workspace)

    def _norm_backward(self, dN, d_out, dx, d_norm_w, d_b_o, parts=None) -> None:
        """The NORM phase on the summed dN, or with ``parts`` (the shards'
        partials of dN) summed by the RMSNorm backward as it reads them."""
        kw = dict(d_normed_parts=parts) if parts else dict(d_normed=dN)
        L.tp_attn_backward(self._desc(), L.BWD_NORM, stream=self.stream, x=self.x, rstd=self.rstd, norm_w=self.norm_w,
                           d_out=d_out, d_x=dx, d_norm_w=d_norm_w, d_b_o=d_b_o, workspace=self.workspace, **kw)

    def materialize_dN(self) -> None:
        """Write the summed dN into its buffer when the step streamed the
        shards' partials into the RMSNorm backward instead (tp_partial_sum:
        the same sum, in the same order, so the same bits the backward used)."""
        if self._dN_streamed:
            L.tp_partial_sum([sh["dN_part"] for sh in self.shards], self.T, self.H, None, None, L.F32, self.dN, L.F32,
                             stream=self.stream)
        self._dN_streamed = False

    def backward(self, mode: str = "equivalence") -> None:
        T, H = self.T, self.H
        fwd_abl = mode == "missing_forward_reduce" and not self.fuse
        outs = self._abl["out"] if fwd_abl else [self.out] * len(self.shards)
        for sh, o in zip(self.shards, outs):
            self._shard_backward(sh, o)
        if mode == "equivalence" or self.fuse:
            # the backward boundary: the shards' partials summed inside the RMSNorm backward
            parts = None if self.fuse else [sh["dN_part"] for sh in self.shards]
            self._norm_backward(self.dN, self.out, self.dx, self.d_norm_w, self.d_b_o, parts=parts)
            self._dN_streamed = not self.fuse
            return
        if mode != "missing_backward_reduce":
            L.tp_partial_sum([sh["dN_part"] for sh in self.shards], T, H, None, None, L.F32, self.dN, L.F32,
                             stream=self.stream)
        dxs = self._abl_bufs("dx", (T, H), torch.bfloat16)
        dws = self._abl_bufs("d_norm_w", (H,), torch.float32)
        dbs = self._abl_bufs("d_b_o", (H,), torch.float32)
        for s, sh in enumerate(self.shards):
            self._norm_backward(self.dN if fwd_abl else sh["dN_part"], outs[s], dxs[s], dws[s], dbs[s])

    def sgd(self) -> None:
        lst = [(t, self.new[n], self._grad_of(n), None, None, t.numel()) for n, t in self._param_list()]
        L.tp_mlp_sgd_step_multi(lst, L.BF16, self.w.lr, stream=self.stream)

    def step(self, mode: str = "equivalence", update: bool = True) -> None:
        if mode not in self.MODES:
            raise ValueError(mode)
        self.forward(mode)
        self.backward(mode)
        if update and mode == "equivalence":
            self.sgd()

    def results(self, mode: str = "equivalence") -> dict:
        """CPU copies (float32) with the shards' slices placed back into the dense w_qkv rows and w_o columns."""
        self.materialize_dN()
        c = lambda t: t.detach().float().cpu()
        w, D = self.w, self.D
        W_full = (w.n_q + 2 * w.n_kv) * D
        r = {"normed": c(self.normed), "rstd": c(self.rstd)}
        dq = torch.zeros(W_full, self.H)
        do = torch.zeros(self.H, w.n_q * D)
        nq_ = torch.zeros(W_full, self.H)
        no_ = torch.zeros(self.H, w.n_q * D)
        for s, sh in enumerate(self.shards):
            dq[sh["rows"]] = c(sh["d_w_qkv"])
            nq_[sh["rows"]] = c(self.new[f"w_qkv.{s}"])
            cols = slice(s * self.nq * D, (s + 1) * self.nq * D)
            do[:, cols] = c(sh["d_w_o"])
            no_[:, cols] = c(self.new[f"w_o.{s}"])
        r.update(d_w_qkv=dq, d_w_o=do, new_w_qkv=nq_, new_w_o=no_, new_norm_w=c(self.new["norm_w"]),
                 new_b_o=c(self.new["b_o"]))
        r["attn_out"] = torch.cat([c(sh["attn_out"]) for sh in self.shards], dim=1)
        if mode == "equivalence" or self.fuse:
            r.update(out=c(self.out), dx=c(self.dx), d_norm_w=c(self.d_norm_w), d_b_o=c(self.d_b_o), dN=c(self.dN))
        else:
            r["out"] = [c(o) for o in self._abl["out"]] if mode == "missing_forward_reduce" else c(self.out)
            r["dx"] = [c(t) for t in self._abl["dx"]]
            r["d_norm_w"] = [c(t) for t in self._abl["d_norm_w"]]
            r["d_b_o"] = [c(t) for t in self._abl["d_b_o"]]
        return r
