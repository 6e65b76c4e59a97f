"""Seeded synthetic inputs for the tensor-parallel MLP sublayer.

This module is shared by the oracle side (tests, the CPU baseline) and the
GPU side (tests, bench).  It holds only the workload table and the random
draws; none of the method's arithmetic lives here.

Workloads
---------
The block is the pre-RMSNorm SwiGLU MLP sublayer rebuilt in "Megatron
tensor-parallel MLP" (synapticradio.com), section "Start with the dense
block": a norm weight [H] (initialised to ones), a stacked gate/up weight
[2, F, H] (plane 0 = gate, plane 1 = up), a down weight [H, F] and a down
bias [H] (initialised to zeros).  The GeLU variant is the classic Megatron
MLP of "Megatron-LM walkthrough", Part II (fc1 [F, H] with bias [F], GeLU,
fc2 [H, F] with bias [H]).

Draw order (fixed, so the oracle and the GPU read identical values):
  1. x ~ N(0, 1) of shape [T, H], fp32;
  2. outlier rows (only where ``outlier_frac > 0``): k = round(frac * T) rows
     picked by ``randperm(T)[:k]`` from the same generator, scaled by
     ``outlier_scale``;
  3. the expansion weight (gate/up [2, F_full, H] or fc1 [F_full, H]) ~ N(0, w_std);
  4. the down weight [H, F_full] ~ N(0, w_std);
  5. norm weight = 1, biases = 0 (the module initialisation on the page);
  6. only when ``perturb=True``: norm weight += 0.1 N(0,1), biases = 0.1 N(0,1)
     (drawn after everything above, so steps 1-4 are unchanged).  Parity tests
     use this to exercise the weight and bias terms that ones/zeros hide.
Everything is drawn in fp32 with ``torch.Generator().manual_seed(seed)`` on
the CPU; bf16 workloads then round every tensor once to bf16 (round to
nearest even, torch's conversion).  Both sides consume those rounded values.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "workload", "draw", "shard_slices", "small_workload", "AttnWorkload",
           "ATTN_WORKLOADS", "attn_workload", "draw_attn"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    tokens: int          # T = batch * seq, rows of the flattened [T, H] activation
    hidden: int          # H
    ffn_full: int        # F_full, the dense FFN width before sharding
    shards: int          # S, the tensor-parallel degree emulated in sequence
    act: str             # "swiglu" | "gelu"
    dtype: str           # "fp32" | "bf16": storage type of weights and activations
    w_std: float
    seed: int
    lr: float = 0.1
    eps: float = 1e-6
    outlier_frac: float = 0.0
    outlier_scale: float = 50.0
    master: bool = False  # fp32 master weights for the SGD update
    shards_run: Optional[int] = None  # how many of the S shards are run (None: all)
    batch: int = 0
    seq: int = 0

    @property
    def ffn_local(self) -> int:
        return self.ffn_full // self.shards

    @property
    def n_run(self) -> int:
        return self.shards if self.shards_run is None else self.shards_run

    @property
    def flops_per_shard(self) -> int:
        """Algorithmic GEMM flops of one shard's forward + backward."""
        mult = 18 if self.act == "swiglu" else 12
        return mult * self.tokens * self.hidden * self.ffn_local

    @property
    def flops_per_step(self) -> int:
        return self.flops_per_shard * self.n_run


# The five workloads.  Shapes follow the model families the workload table
# names (GPT-2 small, Llama-3-8B, Llama-3-70B); the data is synthetic.
WORKLOADS = {
    "tiny_fp32_tp2": Workload("tiny_fp32_tp2", tokens=4, hidden=8, ffn_full=16, shards=2,
                              act="swiglu", dtype="fp32", w_std=0.02, seed=0, batch=1, seq=4),
    "gpt2s_gelu_tp1": Workload("gpt2s_gelu_tp1", tokens=4096, hidden=768, ffn_full=3072,
                               shards=1, act="gelu", dtype="bf16", w_std=0.02, seed=1,
                               batch=4, seq=1024),
    "llama3_8b_tp8": Workload("llama3_8b_tp8", tokens=8192, hidden=4096, ffn_full=14336,
                              shards=8, act="swiglu", dtype="bf16", w_std=0.02, seed=2,
                              batch=2, seq=4096),
    # One rank of TP=8 run as a self-contained block with F = 28672 / 8.
    "llama3_70b_tp8_rank": Workload("llama3_70b_tp8_rank", tokens=16384, hidden=8192,
                                    ffn_full=3584, shards=1, act="swiglu", dtype="bf16",
                                    w_std=0.01, seed=3, batch=4, seq=4096),
    "llama3_8b_tp1_master": Workload("llama3_8b_tp1_master", tokens=32768, hidden=4096,
                                     ffn_full=14336, shards=1, act="swiglu", dtype="bf16",
                                     w_std=0.02, seed=4, outlier_frac=0.01, master=True,
                                     batch=8, seq=4096),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def small_workload(base: Workload, tokens: int, hidden: int, ffn_full: int,
                   shards: Optional[int] = None, **kw) -> Workload:
    """A reduced-size copy of ``base`` (same act, dtype, std, seed)."""
    return dataclasses.replace(base, name=f"{base.name}_T{tokens}H{hidden}F{ffn_full}",
                               tokens=tokens, hidden=hidden, ffn_full=ffn_full,
                               shards=base.shards if shards is None else shards, **kw)


def _round(t: torch.Tensor, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype == "fp32":
        return t.contiguous()
    raise ValueError(dtype)


def draw(w: Workload, perturb: bool = False) -> dict:
    """Draw the dense tensors of workload ``w`` (CPU torch tensors).

    Returns a dict with x [T,H], norm_w [H], w_in ([2,F_full,H] or [F_full,H]),
    b_in ([F_full] for GeLU, else None), w_down [H,F_full], b_down [H], and
    ``outlier_rows`` (LongTensor, possibly empty).  Tensors are in the
    workload's storage dtype.
    """
    g = torch.Generator().manual_seed(w.seed)
    T, H, F = w.tokens, w.hidden, w.ffn_full
    x = torch.randn(T, H, generator=g, dtype=torch.float32)
    rows = torch.empty(0, dtype=torch.long)
    if w.outlier_frac > 0 and T > 0:
        k = int(round(w.outlier_frac * T))
        rows = torch.randperm(T, generator=g)[:k]
        x[rows] *= w.outlier_scale
    if w.act == "swiglu":
        w_in = torch.randn(2, F, H, generator=g, dtype=torch.float32) * w.w_std
    else:
        w_in = torch.randn(F, H, generator=g, dtype=torch.float32) * w.w_std
    w_down = torch.randn(H, F, generator=g, dtype=torch.float32) * w.w_std
    norm_w = torch.ones(H, dtype=torch.float32)
    b_down = torch.zeros(H, dtype=torch.float32)
    b_in = torch.zeros(F, dtype=torch.float32) if w.act == "gelu" else None
    if perturb:
        norm_w += 0.1 * torch.randn(H, generator=g, dtype=torch.float32)
        b_down = 0.1 * torch.randn(H, generator=g, dtype=torch.float32)
        if b_in is not None:
            b_in = 0.1 * torch.randn(F, generator=g, dtype=torch.float32)
    out = dict(x=x, norm_w=norm_w, w_in=w_in, b_in=b_in, w_down=w_down, b_down=b_down)
    out = {k: (None if v is None else _round(v, w.dtype)) for k, v in out.items()}
    out["outlier_rows"] = rows
    return out


def shard_slices(w: Workload, s: int) -> tuple:
    """FFN interval [lo, hi) owned by shard s: contiguous blocks of F_full/S
    channels, the same interval for gate rows, up rows and down columns."""
    if w.ffn_full % w.shards:
        raise ValueError("ffn_full must be divisible by shards")
    fl = w.ffn_full // w.shards
    return s * fl, (s + 1) * fl


def to_numpy64(t: Optional[torch.Tensor]) -> Optional[np.ndarray]:
    """Exact upcast of a CPU tensor (fp32 or bf16) to a float64 numpy array."""
    if t is None:
        return None
    return t.detach().to(torch.float64).cpu().numpy()


# ---------------------------------------------------------------- attention

@dataclasses.dataclass(frozen=True)
class AttnWorkload:
    """The attention sublayer: x [batch, seq, H] flattened to [T, H]; n_q
    query heads and n_kv key/value heads of width d over S tensor-parallel
    shards (each shard: complete query/KV groups)."""
    name: str
    batch: int
    seq: int
    hidden: int
    n_q: int
    n_kv: int
    d: int
    shards: int
    w_std: float
    seed: int
    lr: float = 0.1
    eps: float = 1e-6
    dtype: str = "bf16"

    @property
    def tokens(self) -> int:
        return self.batch * self.seq

    @property
    def flops_per_step(self) -> int:
        """Algorithmic flops of one step over all shards: the four projections
        (forward and backward, 6 flops per weight per token) plus causal
        attention (forward 2 matmuls, backward 4, each over the s(s+1)/2
        query-key pairs of a sequence)."""
        T, H, D = self.tokens, self.hidden, self.d
        W = (self.n_q + 2 * self.n_kv) * D
        proj = 6 * T * H * (W + self.n_q * D)
        pairs = self.batch * self.seq * (self.seq + 1) // 2
        attn = 6 * 2 * pairs * D * self.n_q
        return proj + attn


ATTN_WORKLOADS = {
    "attn_llama3_8b_tp8": AttnWorkload("attn_llama3_8b_tp8", batch=2, seq=4096, hidden=4096, n_q=32, n_kv=8, d=128,
                                       shards=8, w_std=0.02, seed=12),
    "attn_gpt2s_tp1": AttnWorkload("attn_gpt2s_tp1", batch=4, seq=1024, hidden=768, n_q=12, n_kv=12, d=64, shards=1,
                                   w_std=0.02, seed=11),
}


def attn_workload(name: str) -> AttnWorkload:
    return ATTN_WORKLOADS[name]


def draw_attn(w: AttnWorkload, perturb: bool = False) -> dict:
    """Dense tensors of an attention workload (CPU torch tensors, storage dtype):
    x [T, H] ~ N(0,1); w_qkv [(n_q + 2 n_kv) d, H] ~ N(0, std) (rows: Q heads,
    K heads, V heads); w_o [H, n_q d] ~ N(0, std); norm_w = 1, b_o = 0, then
    (perturb) norm_w += 0.1 N(0,1), b_o = 0.1 N(0,1).  Drawn in that order."""
    g = torch.Generator().manual_seed(w.seed)
    T, H, D = w.tokens, w.hidden, w.d
    x = torch.randn(T, H, generator=g, dtype=torch.float32)
    w_qkv = torch.randn((w.n_q + 2 * w.n_kv) * D, H, generator=g, dtype=torch.float32) * w.w_std
    w_o = torch.randn(H, w.n_q * D, generator=g, dtype=torch.float32) * w.w_std
    norm_w = torch.ones(H, dtype=torch.float32)
    b_o = torch.zeros(H, dtype=torch.float32)
    if perturb:
        norm_w += 0.1 * torch.randn(H, generator=g, dtype=torch.float32)
        b_o = 0.1 * torch.randn(H, generator=g, dtype=torch.float32)
    out = dict(x=x, norm_w=norm_w, w_qkv=w_qkv, w_o=w_o, b_o=b_o)
    return {k: _round(v, w.dtype) for k, v in out.items()}

