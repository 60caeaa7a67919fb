"""PyTorch-facing wrapper of the C ABI: device buffers, streams and autograd.

Argument marshalling only: shapes are checked and flattened, outputs and
workspaces are allocated with torch on the inputs' device, pointers and the
current HIP stream are passed to libflp.so.  Nothing here computes any part of
the operator.

Semantics ("Fused Linear LogP" docs page, sections "Entry Point" and "Tensor
Contract"): hidden [B, S, D] or [N, D], weight [V, D], targets [B, S] or [N]
(int64 or int32), optional float32 bias [V]; hidden and weight bfloat16, float16 or
float32; output float32 with the leading
shape of targets.  The optional per-row temperature [B, S] / [N] divides the
logits of its row (PR #555 summary).  Gradients flow to hidden, weight and bias;
targets and temperature are not differentiable.
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch

from . import _abi
from ._abi import FLP_BF16, FLP_F16, FLP_F32, FLP_I32, FLP_I64, FLP_OK, FlpError

# Default cap on the backward workspace: a larger workspace only means larger row
# chunks (same bits); 16 GiB keeps a whole 16384-row chunk of dz and dz^T.
DEFAULT_BWD_WORKSPACE = 16 << 30

_X_DTYPES = {torch.bfloat16: FLP_BF16, torch.float16: FLP_F16, torch.float32: FLP_F32}
_T_DTYPES = {torch.int64: FLP_I64, torch.int32: FLP_I32}


def _ptr(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else int(t.data_ptr())


def _stream(device: torch.device) -> int:
    return int(torch.cuda.current_stream(device).cuda_stream)


def _check(fn: str, status: int) -> None:
    if status != FLP_OK:
        raise FlpError(fn, status)


def _prepare(hidden, weight, targets, bias, temperature):
    if hidden.dtype not in _X_DTYPES or weight.dtype != hidden.dtype:
        raise TypeError("hidden and weight must have the same dtype: bfloat16, float16 or float32")
    if targets.dtype not in _T_DTYPES:
        raise TypeError("targets must be int64 or int32")
    if not (hidden.is_cuda and weight.is_cuda and targets.is_cuda):
        raise ValueError("hidden, weight and targets must be on the GPU")
    for name, t in (("hidden", hidden), ("weight", weight), ("targets", targets),
                    ("bias", bias), ("temperature", temperature)):
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if weight.dim() != 2 or hidden.shape[-1] != weight.shape[1]:
        raise ValueError("weight must be [V, D] with D = hidden.shape[-1]")
    lead = tuple(targets.shape)
    if tuple(hidden.shape[:-1]) != lead:
        raise ValueError("hidden leading shape must equal the targets shape")
    D = int(hidden.shape[-1])
    V = int(weight.shape[0])
    h2 = hidden.reshape(-1, D)
    t1 = targets.reshape(-1)
    N = int(t1.shape[0])
    if bias is not None and (bias.dtype != torch.float32 or tuple(bias.shape) != (V,)):
        raise ValueError("bias must be float32 [V]")
    temp1 = None
    if temperature is not None:
        if temperature.dtype != torch.float32 or tuple(temperature.shape) != lead:
            raise ValueError("temperature must be float32 with the targets shape")
        temp1 = temperature.reshape(-1)
    return h2, t1, temp1, lead, N, D, V


def forward(hidden: torch.Tensor, weight: torch.Tensor, targets: torch.Tensor,
            bias: Optional[torch.Tensor] = None, temperature: Optional[torch.Tensor] = None,
            return_lse: bool = True, workspace: Optional[torch.Tensor] = None
            ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """logp (and lse) float32 with the targets' leading shape, through flp_forward."""
    h2, t1, temp1, lead, N, D, V = _prepare(hidden, weight, targets, bias, temperature)
    dev = hidden.device
    logp = torch.empty(lead, dtype=torch.float32, device=dev)
    lse = torch.empty(lead, dtype=torch.float32, device=dev) if return_lse else None
    need = _abi.flp_forward_workspace_bytes(N, D, V)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    st = _abi.flp_forward(N, D, V, _X_DTYPES[hidden.dtype], _ptr(h2), _ptr(weight), _ptr(bias),
                          _ptr(t1), _T_DTYPES[targets.dtype], _ptr(temp1), _ptr(logp), _ptr(lse),
                          _ptr(workspace), workspace.numel() * workspace.element_size(),
                          _stream(dev))
    _check("flp_forward", st)
    return logp, lse


def forward_partial(hidden: torch.Tensor, weight_shard: torch.Tensor, targets: torch.Tensor,
                    vocab_start: int, vocab_size: int, bias_shard: Optional[torch.Tensor] = None,
                    temperature: Optional[torch.Tensor] = None
                    ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Per-tile (max, sum-of-exp) partials [ceil(V_local / 256), N, 2] and the zt [N] of one
    vocabulary shard (rows vocab_start .. vocab_start + V_local - 1 of the weight), through
    flp_forward_partial.  Targets are global ids; vocab_size is the full vocabulary."""
    h2, t1, temp1, lead, N, D, V_local = _prepare(hidden, weight_shard, targets, bias_shard,
                                                  temperature)
    dev = hidden.device
    partial = torch.empty(((V_local + 255) // 256, N, 2), dtype=torch.float32, device=dev)
    zt = torch.empty(N, dtype=torch.float32, device=dev)
    st = _abi.flp_forward_partial(N, D, V_local, int(vocab_start), int(vocab_size),
                                  _X_DTYPES[hidden.dtype], _ptr(h2), _ptr(weight_shard),
                                  _ptr(bias_shard), _ptr(t1), _T_DTYPES[targets.dtype],
                                  _ptr(temp1), _ptr(partial), _ptr(zt), _stream(dev))
    _check("flp_forward_partial", st)
    return partial, zt


def merge(partials: torch.Tensor, zt: torch.Tensor, targets: torch.Tensor, vocab_size: int,
          return_lse: bool = True) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """logp (and lse) from the shards' partials concatenated in ascending vocabulary order
    ([ceil(vocab_size / 256), N, 2]) and the sum of their zt, through flp_merge."""
    if targets.dtype not in _T_DTYPES:
        raise TypeError("targets must be int64 or int32")
    lead = tuple(targets.shape)
    t1 = targets.reshape(-1)
    N = int(t1.shape[0])
    n_vt = (int(vocab_size) + 255) // 256
    if (partials.dtype != torch.float32 or tuple(partials.shape) != (n_vt, N, 2)
            or not partials.is_contiguous()):
        raise ValueError(f"partials must be contiguous float32 [{n_vt}, {N}, 2]")
    if zt.dtype != torch.float32 or tuple(zt.shape) != (N,) or not zt.is_contiguous():
        raise ValueError("zt must be contiguous float32 [N]")
    if not t1.is_contiguous():
        raise ValueError("targets must be contiguous")
    dev = partials.device
    logp = torch.empty(lead, dtype=torch.float32, device=dev)
    lse = torch.empty(lead, dtype=torch.float32, device=dev) if return_lse else None
    st = _abi.flp_merge(N, int(vocab_size), _ptr(partials), _ptr(zt), _ptr(t1),
                        _T_DTYPES[targets.dtype], _ptr(logp), _ptr(lse), _stream(dev))
    _check("flp_merge", st)
    return logp, lse


def backward_workspace_bytes(N: int, D: int, V: int, x_dtype: torch.dtype,
                             dw_dtype: Optional[torch.dtype] = None, chunk_rows: int = 0) -> int:
    dw = _X_DTYPES[x_dtype if dw_dtype is None else dw_dtype]
    return _abi.flp_backward_workspace_bytes(N, D, V, _X_DTYPES[x_dtype], dw, chunk_rows)


def default_backward_workspace_bytes(N: int, D: int, V: int, x_dtype: torch.dtype,
                                     dw_dtype: Optional[torch.dtype] = None,
                                     cap: int = DEFAULT_BWD_WORKSPACE) -> int:
    """The whole batch as one chunk if that fits under ``cap``, else the minimum
    plus as many 256-row quanta as fit (same bits either way)."""
    full = backward_workspace_bytes(N, D, V, x_dtype, dw_dtype, chunk_rows=max(N, 1))
    if full <= cap:
        return full
    lo = backward_workspace_bytes(N, D, V, x_dtype, dw_dtype, chunk_rows=0)
    return max(lo, cap)


def backward(grad_out: torch.Tensor, lse: torch.Tensor, hidden: torch.Tensor, weight: torch.Tensor,
             targets: torch.Tensor, bias: Optional[torch.Tensor] = None,
             temperature: Optional[torch.Tensor] = None, need_hidden: bool = True,
             need_weight: bool = True, need_bias: Optional[bool] = None,
             dw_dtype: Optional[torch.dtype] = None, workspace_bytes: Optional[int] = None,
             workspace: Optional[torch.Tensor] = None):
    """(d_hidden, d_weight, d_bias) through flp_backward; unrequested ones are None."""
    h2, t1, temp1, lead, N, D, V = _prepare(hidden, weight, targets, bias, temperature)
    dev = hidden.device
    if need_bias is None:
        need_bias = bias is not None
    if grad_out.dtype != torch.float32 or tuple(grad_out.shape) != lead or not grad_out.is_contiguous():
        raise ValueError("grad_out must be contiguous float32 with the targets shape")
    if lse.dtype != torch.float32 or tuple(lse.shape) != lead or not lse.is_contiguous():
        raise ValueError("lse must be contiguous float32 with the targets shape")
    dwt = hidden.dtype if dw_dtype is None else dw_dtype
    d_hidden = torch.empty_like(hidden) if need_hidden else None
    d_weight = torch.empty(weight.shape, dtype=dwt, device=dev) if need_weight else None
    d_bias = torch.empty(V, dtype=torch.float32, device=dev) if need_bias else None
    if workspace is None:
        if workspace_bytes is None:
            workspace_bytes = default_backward_workspace_bytes(N, D, V, hidden.dtype, dwt)
        workspace = torch.empty(max(int(workspace_bytes), 16), dtype=torch.uint8, device=dev)
    st = _abi.flp_backward(N, D, V, _X_DTYPES[hidden.dtype], _ptr(grad_out), _ptr(lse), _ptr(h2),
                           _ptr(weight), _ptr(bias), _ptr(t1), _T_DTYPES[targets.dtype],
                           _ptr(temp1), _ptr(d_hidden), _ptr(d_weight), _X_DTYPES[dwt],
                           _ptr(d_bias), _ptr(workspace),
                           workspace.numel() * workspace.element_size(), _stream(dev))
    _check("flp_backward", st)
    return d_hidden, d_weight, d_bias


class LinearLogp(torch.autograd.Function):
    """Autograd node: the forward saves lse; the backward recomputes the logits."""

    @staticmethod
    def forward(ctx, hidden, weight, targets, bias, temperature):
        logp, lse = forward(hidden, weight, targets, bias, temperature, return_lse=True)
        ctx.save_for_backward(hidden, weight, targets, bias, temperature, lse)
        ctx.mark_non_differentiable(lse)
        return logp, lse

    @staticmethod
    def backward(ctx, g_logp, g_lse):
        hidden, weight, targets, bias, temperature, lse = ctx.saved_tensors
        need_h, need_w, _, need_b, _ = ctx.needs_input_grad
        if not (need_h or need_w or need_b):
            return None, None, None, None, None
        g = g_logp.contiguous().to(torch.float32)
        dh, dw, db = backward(g, lse, hidden, weight, targets, bias, temperature,
                              need_hidden=need_h, need_weight=need_w,
                              need_bias=bool(need_b and bias is not None))
        return dh, dw, None, db, None


def linear_logp_with_lse(hidden, weight, targets, bias=None, temperature=None):
    """(logp, lse): selected-token log-probabilities and the per-row log-sum-exp."""
    return LinearLogp.apply(hidden, weight, targets, bias, temperature)


def linear_logp(hidden, weight, targets, bias=None, temperature=None):
    """logp[..] = log_softmax((hidden @ weight^T + bias) / T)[target], 0 for out-of-range targets."""
    return linear_logp_with_lse(hidden, weight, targets, bias, temperature)[0]


# ---- the operator on materialised logits ------------------------------------------------------

def _prepare_logits(logits, targets):
    if logits.dtype not in _X_DTYPES:
        raise TypeError("logits must be bfloat16, float16 or float32")
    if targets.dtype not in _T_DTYPES:
        raise TypeError("targets must be int64 or int32")
    if not (logits.is_cuda and targets.is_cuda):
        raise ValueError("logits and targets must be on the GPU")
    if not (logits.is_contiguous() and targets.is_contiguous()):
        raise ValueError("logits and targets must be contiguous")
    lead = tuple(targets.shape)
    if tuple(logits.shape[:-1]) != lead:
        raise ValueError("logits leading shape must equal the targets shape")
    V = int(logits.shape[-1])
    t1 = targets.reshape(-1)
    return logits.reshape(-1, V), t1, lead, int(t1.shape[0]), V


def logits_forward(logits: torch.Tensor, targets: torch.Tensor, return_lse: bool = True
                   ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """logp (and lse) of given logits [.., V] through flp_logits_forward."""
    z2, t1, lead, N, V = _prepare_logits(logits, targets)
    dev = logits.device
    logp = torch.empty(lead, dtype=torch.float32, device=dev)
    lse = torch.empty(lead, dtype=torch.float32, device=dev) if return_lse else None
    st = _abi.flp_logits_forward(N, V, _X_DTYPES[logits.dtype], _ptr(z2), _ptr(t1),
                                 _T_DTYPES[targets.dtype], _ptr(logp), _ptr(lse), _stream(dev))
    _check("flp_logits_forward", st)
    return logp, lse


def logits_backward(grad_out: torch.Tensor, lse: torch.Tensor, logits: torch.Tensor,
                    targets: torch.Tensor) -> torch.Tensor:
    """d logits (logits dtype) through flp_logits_backward."""
    z2, t1, lead, N, V = _prepare_logits(logits, targets)
    for name, x in (("grad_out", grad_out), ("lse", lse)):
        if x.dtype != torch.float32 or tuple(x.shape) != lead or not x.is_contiguous():
            raise ValueError(f"{name} must be contiguous float32 with the targets shape")
    d = torch.empty_like(logits)
    st = _abi.flp_logits_backward(N, V, _X_DTYPES[logits.dtype], _ptr(grad_out), _ptr(lse),
                                  _ptr(z2), _ptr(t1), _T_DTYPES[targets.dtype], _ptr(d),
                                  _stream(logits.device))
    _check("flp_logits_backward", st)
    return d


class LogitsLogp(torch.autograd.Function):
    """Autograd node of the operator on materialised logits; the forward saves lse."""

    @staticmethod
    def forward(ctx, logits, targets):
        logp, lse = logits_forward(logits, targets, return_lse=True)
        ctx.save_for_backward(logits, targets, lse)
        return logp

    @staticmethod
    def backward(ctx, g_logp):
        logits, targets, lse = ctx.saved_tensors
        if not ctx.needs_input_grad[0]:
            return None, None
        return logits_backward(g_logp.contiguous().to(torch.float32), lse, logits, targets), None


def logits_logp(logits, targets):
    """logp[..] = log_softmax(logits)[target], 0 for out-of-range targets (differentiable)."""
    return LogitsLogp.apply(logits, targets)


# ---- indexed (row-subset) variants ------------------------------------------------------------
#
# rows: 1-D int64 / int32 ids into the flattened batch (PR #547 "What", indexed
# semantics): outputs keep the full row shape, a duplicated id selects its row
# once, ids outside [0, N) are ignored, rows left out get logp = lse = 0 and zero
# gradients; d_weight and d_bias sum over the selected rows.

def _prepare_rows(rows: torch.Tensor, dev: torch.device):
    if rows.dtype not in _T_DTYPES:
        raise TypeError("rows must be int64 or int32")
    if rows.dim() != 1 or not rows.is_contiguous() or rows.device != dev:
        raise ValueError("rows must be a contiguous 1-D tensor on the inputs' device")
    return rows, int(rows.shape[0]), _T_DTYPES[rows.dtype]


def forward_indexed(hidden: torch.Tensor, weight: torch.Tensor, targets: torch.Tensor,
                    rows: torch.Tensor, bias: Optional[torch.Tensor] = None,
                    temperature: Optional[torch.Tensor] = None, return_lse: bool = True
                    ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """logp (and lse) of the selected rows, zeros elsewhere, through flp_forward_indexed."""
    h2, t1, temp1, lead, N, D, V = _prepare(hidden, weight, targets, bias, temperature)
    dev = hidden.device
    rows, n_rows, r_dt = _prepare_rows(rows, dev)
    logp = torch.empty(lead, dtype=torch.float32, device=dev)
    lse = torch.empty(lead, dtype=torch.float32, device=dev) if return_lse else None
    need = _abi.flp_forward_indexed_workspace_bytes(N, D, V, _X_DTYPES[hidden.dtype], n_rows)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    st = _abi.flp_forward_indexed(N, D, V, _X_DTYPES[hidden.dtype], _ptr(h2), _ptr(weight),
                                  _ptr(bias), _ptr(t1), _T_DTYPES[targets.dtype], _ptr(temp1),
                                  _ptr(rows), r_dt, n_rows, _ptr(logp), _ptr(lse), _ptr(ws),
                                  ws.numel(), _stream(dev))
    _check("flp_forward_indexed", st)
    return logp, lse


def backward_indexed(grad_out: torch.Tensor, lse: torch.Tensor, hidden: torch.Tensor,
                     weight: torch.Tensor, targets: torch.Tensor, rows: torch.Tensor,
                     bias: Optional[torch.Tensor] = None,
                     temperature: Optional[torch.Tensor] = None, need_hidden: bool = True,
                     need_weight: bool = True, need_bias: Optional[bool] = None,
                     dw_dtype: Optional[torch.dtype] = None,
                     workspace_bytes: Optional[int] = None):
    """(d_hidden, d_weight, d_bias) of the selected rows through flp_backward_indexed."""
    h2, t1, temp1, lead, N, D, V = _prepare(hidden, weight, targets, bias, temperature)
    dev = hidden.device
    rows, n_rows, r_dt = _prepare_rows(rows, dev)
    if need_bias is None:
        need_bias = bias is not None
    for name, x in (("grad_out", grad_out), ("lse", lse)):
        if x.dtype != torch.float32 or tuple(x.shape) != lead or not x.is_contiguous():
            raise ValueError(f"{name} must be contiguous float32 with the targets shape")
    dwt = hidden.dtype if dw_dtype is None else dw_dtype
    xd, wd = _X_DTYPES[hidden.dtype], _X_DTYPES[dwt]
    d_hidden = torch.empty_like(hidden) if need_hidden else None
    d_weight = torch.empty(weight.shape, dtype=dwt, device=dev) if need_weight else None
    d_bias = torch.empty(V, dtype=torch.float32, device=dev) if need_bias else None
    if workspace_bytes is None:
        cap = max(min(n_rows, N), 1)
        workspace_bytes = _abi.flp_backward_indexed_workspace_bytes(N, D, V, xd, wd, n_rows, cap)
        if workspace_bytes > DEFAULT_BWD_WORKSPACE:
            workspace_bytes = max(DEFAULT_BWD_WORKSPACE,
                                  _abi.flp_backward_indexed_workspace_bytes(N, D, V, xd, wd,
                                                                            n_rows, 0))
    ws = torch.empty(max(int(workspace_bytes), 16), dtype=torch.uint8, device=dev)
    st = _abi.flp_backward_indexed(N, D, V, xd, _ptr(grad_out), _ptr(lse), _ptr(h2),
                                   _ptr(weight), _ptr(bias), _ptr(t1), _T_DTYPES[targets.dtype],
                                   _ptr(temp1), _ptr(rows), r_dt, n_rows, _ptr(d_hidden),
                                   _ptr(d_weight), wd, _ptr(d_bias), _ptr(ws), ws.numel(),
                                   _stream(dev))
    _check("flp_backward_indexed", st)
    return d_hidden, d_weight, d_bias


class LinearLogpIndexed(torch.autograd.Function):
    """Autograd node of the indexed linear operator; the forward saves lse."""

    @staticmethod
    def forward(ctx, hidden, weight, targets, rows, bias, temperature):
        logp, lse = forward_indexed(hidden, weight, targets, rows, bias, temperature)
        ctx.save_for_backward(hidden, weight, targets, rows, bias, temperature, lse)
        ctx.mark_non_differentiable(lse)
        return logp, lse

    @staticmethod
    def backward(ctx, g_logp, g_lse):
        hidden, weight, targets, rows, bias, temperature, lse = ctx.saved_tensors
        need_h, need_w, _, _, need_b, _ = ctx.needs_input_grad
        if not (need_h or need_w or need_b):
            return None, None, None, None, None, None
        dh, dw, db = backward_indexed(g_logp.contiguous().to(torch.float32), lse, hidden, weight,
                                      targets, rows, bias, temperature, need_hidden=need_h,
                                      need_weight=need_w,
                                      need_bias=bool(need_b and bias is not None))
        return dh, dw, None, None, db, None


def linear_logp_indexed(hidden, weight, targets, rows, bias=None, temperature=None):
    """linear_logp restricted to the rows listed in ``rows`` (full shape, zeros elsewhere)."""
    return LinearLogpIndexed.apply(hidden, weight, targets, rows, bias, temperature)[0]


def logits_forward_indexed(logits: torch.Tensor, targets: torch.Tensor, rows: torch.Tensor,
                           return_lse: bool = True
                           ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """logp (and lse) of the selected rows of given logits through flp_logits_forward_indexed."""
    z2, t1, lead, N, V = _prepare_logits(logits, targets)
    dev = logits.device
    rows, n_rows, r_dt = _prepare_rows(rows, dev)
    logp = torch.empty(lead, dtype=torch.float32, device=dev)
    lse = torch.empty(lead, dtype=torch.float32, device=dev) if return_lse else None
    ws = torch.empty(max(_abi.flp_logits_indexed_workspace_bytes(N), 16), dtype=torch.uint8,
                     device=dev)
    st = _abi.flp_logits_forward_indexed(N, V, _X_DTYPES[logits.dtype], _ptr(z2), _ptr(t1),
                                         _T_DTYPES[targets.dtype], _ptr(rows), r_dt, n_rows,
                                         _ptr(logp), _ptr(lse), _ptr(ws), ws.numel(), _stream(dev))
    _check("flp_logits_forward_indexed", st)
    return logp, lse


def logits_backward_indexed(grad_out: torch.Tensor, lse: torch.Tensor, logits: torch.Tensor,
                            targets: torch.Tensor, rows: torch.Tensor) -> torch.Tensor:
    """d logits of the selected rows (zero rows elsewhere) through flp_logits_backward_indexed."""
    z2, t1, lead, N, V = _prepare_logits(logits, targets)
    dev = logits.device
    rows, n_rows, r_dt = _prepare_rows(rows, dev)
    for name, x in (("grad_out", grad_out), ("lse", lse)):
        if x.dtype != torch.float32 or tuple(x.shape) != lead or not x.is_contiguous():
            raise ValueError(f"{name} must be contiguous float32 with the targets shape")
    d = torch.empty_like(logits)
    ws = torch.empty(max(_abi.flp_logits_indexed_workspace_bytes(N), 16), dtype=torch.uint8,
                     device=dev)
    st = _abi.flp_logits_backward_indexed(N, V, _X_DTYPES[logits.dtype], _ptr(grad_out),
                                          _ptr(lse), _ptr(z2), _ptr(t1), _T_DTYPES[targets.dtype],
                                          _ptr(rows), r_dt, n_rows, _ptr(d), _ptr(ws), ws.numel(),
                                          _stream(dev))
    _check("flp_logits_backward_indexed", st)
    return d


class LogitsLogpIndexed(torch.autograd.Function):
    """Autograd node of the indexed operator on materialised logits."""

    @staticmethod
    def forward(ctx, logits, targets, rows):
        logp, lse = logits_forward_indexed(logits, targets, rows, return_lse=True)
        ctx.save_for_backward(logits, targets, rows, lse)
        return logp

    @staticmethod
    def backward(ctx, g_logp):
        logits, targets, rows, lse = ctx.saved_tensors
        if not ctx.needs_input_grad[0]:
            return None, None, None
        d = logits_backward_indexed(g_logp.contiguous().to(torch.float32), lse, logits, targets,
                                    rows)
        return d, None, None


def logits_logp_indexed(logits, targets, rows):
    """logits_logp restricted to the rows listed in ``rows`` (full shape, zeros elsewhere)."""
    return LogitsLogpIndexed.apply(logits, targets, rows)


# ---- untied embedding lookup -------------------------------------------------------------------
#
# out = weight[ids] (a zero row for ids outside [0, V)); d_weight sums the gradient rows of each
# id in ascending token order in fp32 (PR #555 summary bullets: sorted-segment deterministic
# grad_weight).

def _prepare_embedding(weight, ids):
    if weight.dtype not in _X_DTYPES:
        raise TypeError("weight must be bfloat16, float16 or float32")
    if ids.dtype not in _T_DTYPES:
        raise TypeError("ids must be int64 or int32")
    if not (weight.is_cuda and ids.is_cuda):
        raise ValueError("weight and ids must be on the GPU")
    if weight.dim() != 2 or not weight.is_contiguous() or not ids.is_contiguous():
        raise ValueError("weight must be a contiguous [V, D] tensor and ids contiguous")
    V, D = int(weight.shape[0]), int(weight.shape[1])
    return V, D, ids.reshape(-1), int(ids.numel())


def embedding_forward(weight: torch.Tensor, ids: torch.Tensor) -> torch.Tensor:
    """weight[ids] with the ids' shape + [D], through flp_embedding_forward."""
    V, D, i1, N = _prepare_embedding(weight, ids)
    out = torch.empty(tuple(ids.shape) + (D,), dtype=weight.dtype, device=weight.device)
    st = _abi.flp_embedding_forward(N, D, V, _X_DTYPES[weight.dtype], _ptr(weight), _ptr(i1),
                                    _T_DTYPES[ids.dtype], _ptr(out), _stream(weight.device))
    _check("flp_embedding_forward", st)
    return out


def embedding_backward(grad: torch.Tensor, ids: torch.Tensor, num_embeddings: int,
                       dw_dtype: Optional[torch.dtype] = None) -> torch.Tensor:
    """d_weight [V, D] of sum(grad * weight[ids]) through flp_embedding_backward."""
    if grad.dtype not in _X_DTYPES or not grad.is_contiguous() or not grad.is_cuda:
        raise ValueError("grad must be a contiguous bfloat16 / float16 / float32 GPU tensor")
    if ids.dtype not in _T_DTYPES or not ids.is_contiguous():
        raise ValueError("ids must be contiguous int64 or int32")
    D = int(grad.shape[-1])
    if tuple(grad.shape[:-1]) != tuple(ids.shape):
        raise ValueError("grad must have the ids' shape + [D]")
    N, V = int(ids.numel()), int(num_embeddings)
    dwt = grad.dtype if dw_dtype is None else dw_dtype
    dev = grad.device
    d_weight = torch.empty((V, D), dtype=dwt, device=dev)
    ws = torch.empty(max(_abi.flp_embedding_backward_workspace_bytes(N, D, V), 16),
                     dtype=torch.uint8, device=dev)
    st = _abi.flp_embedding_backward(N, D, V, _X_DTYPES[grad.dtype], _ptr(grad), _ptr(ids),
                                     _T_DTYPES[ids.dtype], _ptr(d_weight), _X_DTYPES[dwt],
                                     _ptr(ws), ws.numel(), _stream(dev))
    _check("flp_embedding_backward", st)
    return d_weight


class Embedding(torch.autograd.Function):
    """Autograd node of the untied embedding lookup; the ids are not differentiable."""

    @staticmethod
    def forward(ctx, weight, ids):
        ctx.save_for_backward(ids)
        ctx.num_embeddings = int(weight.shape[0])
        return embedding_forward(weight, ids)

    @staticmethod
    def backward(ctx, grad):
        (ids,) = ctx.saved_tensors
        if not ctx.needs_input_grad[0]:
            return None, None
        return embedding_backward(grad.contiguous(), ids, ctx.num_embeddings), None


def embedding(weight, ids):
    """weight[ids] (zero rows for ids outside [0, V)), differentiable in weight."""
    return Embedding.apply(weight, ids)
