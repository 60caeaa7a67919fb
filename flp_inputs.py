"""Seeded synthetic inputs for the fused linear log-prob workloads.

Shared by the tests, the benchmark and the smoke check, so that the GPU path
and the CPU oracle see the same tensors.  This module draws random numbers and
lays them out; it holds none of the operator's arithmetic.

The pages measure on the LM head of a released checkpoint whose weights are
not available here, so synthetic tensors of that head's exact shapes
(D = 2688, V = 131072, bf16) stand in for it.  Every tensor is drawn on the
CPU from its own ``torch.Generator`` seeded with ``1000 * cfg + k`` (k = the
tensor's index below), in float32, then rounded to the compute dtype with
round-to-nearest-even (``Tensor.to``).  Independent generators keep W the same
whatever the number of rows drawn.

    k=0 hidden ~ N(0, 1)            [N, D]
    k=1 W      ~ N(0, w_std^2)      [V, D]
    k=2 bias   ~ N(0, bias_std^2)   [V] float32 (when the workload has a bias)
    k=3 targets ~ U{0 .. V-1}       [N] int64
    k=4 ignored-row picks: a random permutation; the first ``n_ignored`` rows
        get the out-of-range ids of ``ignore_values`` in turn
    k=5 temperature ~ U[lo, hi)     [N] float32 (when the workload has one)
    k=6 grad_out: ones, or ~ N(0, 1) [N] float32
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional, Tuple

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    cfg: int
    N: int
    D: int
    V: int
    dtype: torch.dtype
    w_std: float
    bias_std: Optional[float] = None
    n_ignored: int = 0
    ignore_values: Tuple[int, ...] = (-1,)
    temperature: Optional[Tuple[float, float]] = None
    grad: str = "ones"            # "ones" | "normal" | "none" (forward only)
    leading: Tuple[int, ...] = ()
    backward: bool = True

    def with_rows(self, n: int) -> "Workload":
        return replace(self, N=n, leading=(n,), n_ignored=min(self.n_ignored, n))


V_BIG = 131072
WORKLOADS = {
    # tiny fp32 fwd+bwd: parity case the oracle finishes in seconds
    "tiny_fp32": Workload("tiny_fp32", 1, 64, 256, 4096, torch.float32, 0.05, bias_std=0.1,
                          n_ignored=4, ignore_values=(-1,), grad="ones", leading=(64,)),
    # decode-scale forward, memory-bound on streaming W
    "decode_n32": Workload("decode_n32", 2, 32, 2688, V_BIG, torch.bfloat16, 0.02,
                           grad="none", leading=(2, 16), backward=False),
    # rollout-scale forward with per-row temperature
    "rollout_n8192": Workload("rollout_n8192", 3, 8192, 2688, V_BIG, torch.bfloat16, 0.02,
                              temperature=(0.5, 1.5), grad="none", leading=(8, 1024),
                              backward=False),
    # training forward + backward
    "train_n16384": Workload("train_n16384", 4, 16384, 2688, V_BIG, torch.bfloat16, 0.02,
                             bias_std=0.1, grad="normal", leading=(4, 4096)),
    # long-sequence backward stress, 5% out-of-range targets
    "longseq_n65600": Workload("longseq_n65600", 5, 65600, 2688, V_BIG, torch.bfloat16, 0.02,
                               n_ignored=3280, ignore_values=(-1, -100, V_BIG, V_BIG + 12345),
                               grad="ones", leading=(1, 65600)),
}


def _gen(cfg: int, k: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(1000 * cfg + k)
    return g


def draw_hidden(w: Workload) -> torch.Tensor:
    return torch.randn(w.N, w.D, generator=_gen(w.cfg, 0)).to(w.dtype)


def draw_weight(w: Workload) -> torch.Tensor:
    x = torch.randn(w.V, w.D, generator=_gen(w.cfg, 1))
    x.mul_(w.w_std)
    return x.to(w.dtype)


def draw_bias(w: Workload) -> Optional[torch.Tensor]:
    if w.bias_std is None:
        return None
    return torch.randn(w.V, generator=_gen(w.cfg, 2)) * w.bias_std


def draw_targets(w: Workload) -> torch.Tensor:
    t = torch.randint(0, w.V, (w.N,), generator=_gen(w.cfg, 3), dtype=torch.int64)
    if w.n_ignored:
        picks = torch.randperm(w.N, generator=_gen(w.cfg, 4))[: w.n_ignored]
        vals = torch.tensor([w.ignore_values[i % len(w.ignore_values)] for i in range(w.n_ignored)],
                            dtype=torch.int64)
        t[picks] = vals
    return t


def draw_temperature(w: Workload) -> Optional[torch.Tensor]:
    if w.temperature is None:
        return None
    lo, hi = w.temperature
    return torch.rand(w.N, generator=_gen(w.cfg, 5)) * (hi - lo) + lo


def draw_grad(w: Workload) -> Optional[torch.Tensor]:
    if w.grad == "none":
        return None
    if w.grad == "ones":
        return torch.ones(w.N)
    return torch.randn(w.N, generator=_gen(w.cfg, 6))


def make_inputs(name_or_workload, n_rows: Optional[int] = None, weight: Optional[torch.Tensor] = None):
    """All CPU tensors of one workload, as a dict.

    ``n_rows`` overrides N (hidden, targets, temperature and grad_out are drawn
    with that many rows; W and bias do not depend on it).  ``weight`` reuses an
    already drawn W of the same workload (it is large).
    """
    w = WORKLOADS[name_or_workload] if isinstance(name_or_workload, str) else name_or_workload
    if n_rows is not None:
        w = w.with_rows(n_rows)
    out = dict(workload=w, hidden=draw_hidden(w),
               weight=draw_weight(w) if weight is None else weight,
               bias=draw_bias(w), targets=draw_targets(w),
               temperature=draw_temperature(w), grad_out=draw_grad(w))
    return out


def make_logits_inputs(name: str, N: int, V: int, dtype: torch.dtype, seed: int,
                       n_ignored: int = 0, ignore_values=(-1,), logit_std: float = 1.0,
                       grad: str = "normal", device: str = "cpu"):
    """Inputs of the operator on materialised logits: logits ~ N(0, logit_std^2)
    [N, V] in `dtype`, targets (with n_ignored out-of-range rows), grad_out.

    The logits are drawn on `device` from a generator seeded with 1000 * seed
    (large blocks are drawn on the GPU directly; the same seed on the same
    device gives the same tensor); targets, picks and grad_out are drawn on the
    CPU with seeds 1000 * seed + 3, + 4 and + 6, as for the linear workloads.
    """
    w = Workload(name, seed, N, 1, V, dtype, 0.0, n_ignored=n_ignored,
                 ignore_values=tuple(ignore_values), grad=grad, leading=(N,))
    g = torch.Generator(device=device)
    g.manual_seed(1000 * seed)
    z = torch.empty(N, V, dtype=torch.float32, device=device)
    z.normal_(0.0, logit_std, generator=g)
    return dict(workload=w, logits=z.to(dtype), targets=draw_targets(w), grad_out=draw_grad(w))


def make_embedding_inputs(N: int, D: int, V: int, dtype: torch.dtype, seed: int,
                          ids: str = "zipf", invalid: Tuple[int, ...] = (),
                          device: str = "cpu"):
    """Inputs of the untied embedding lookup: a table E ~ N(0, 0.02^2) [V, D] in `dtype`
    (drawn on `device`), token ids [N] int64 and an upstream gradient [N, D] ~ N(0, 1) in
    `dtype`.  ids = "zipf": a heavy-headed token-frequency draw, floor(V^u) - 1 for u
    uniform (many repeats of the frequent ids, most ids absent); "uniform": uniform over
    [0, V); "same": every token has id V // 2.  The given out-of-range values replace
    the first ids (as many as there are tokens)."""
    g = torch.Generator(device=device)
    g.manual_seed(1000 * seed)
    E = torch.empty(V, D, dtype=torch.float32, device=device).normal_(0.0, 0.02, generator=g)
    gc = torch.Generator(device="cpu")
    gc.manual_seed(1000 * seed + 1)
    if ids == "zipf":
        u = torch.rand(N, generator=gc, dtype=torch.float64)
        t = (torch.floor(torch.pow(float(V), u)) - 1).clamp_(0, V - 1).to(torch.int64)
    elif ids == "uniform":
        t = torch.randint(0, V, (N,), generator=gc)
    else:
        t = torch.full((N,), V // 2, dtype=torch.int64)
    k = min(len(invalid), N)
    if k:
        t[:k] = torch.tensor(invalid[:k], dtype=torch.int64)
    grad = torch.empty(N, D, dtype=torch.float32, device=device).normal_(0.0, 1.0, generator=g)
    return dict(weight=E.to(dtype), ids=t, grad=grad.to(dtype))


def random_rows(n_total: int, k: int, seed: int) -> torch.Tensor:
    """A seeded sorted sample of k distinct row indices out of n_total."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return torch.randperm(n_total, generator=g)[:k].sort().values


def row_ids(n_total: int, k: int, seed: int, n_dup: int = 0, invalid: Tuple[int, ...] = (),
            dtype: torch.dtype = torch.int64) -> torch.Tensor:
    """A seeded, shuffled id list for the indexed variants: k distinct rows of n_total,
    n_dup repeats of some of them and the given out-of-range values."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    base = torch.randperm(n_total, generator=g)[:k]
    dup = base[torch.randint(0, max(k, 1), (n_dup,), generator=g)] if k > 0 and n_dup > 0 \
        else torch.empty(0, dtype=torch.int64)
    ids = torch.cat([base, dup, torch.tensor(invalid, dtype=torch.int64)])
    return ids[torch.randperm(ids.numel(), generator=g)].to(dtype).contiguous()


def flops_fwd(N: int, D: int, V: int) -> float:
    """Multiply-adds of the logits contraction, counted as 2 flops each."""
    return 2.0 * N * D * V


def method_flops_fwd_bwd(N: int, D: int, V: int) -> float:
    """Forward + recompute + dX + dW contractions: 4 x 2 N D V."""
    return 8.0 * N * D * V


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


__all__ = ["Workload", "WORKLOADS", "make_inputs", "make_logits_inputs", "random_rows", "flops_fwd",
           "method_flops_fwd_bwd", "ceil_div", "math"]
