"""CPU FP64 oracle for the fused linear selected-token log-probability.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check of the build
entry point and the CPU-baseline leg of the benchmark may import this module.
The GPU library never calls it, and it shares no code with the GPU path.

What it computes (the plain definition, evaluated in float64 on exactly
up-cast inputs, with the [rows, V] logits materialised chunk by chunk):

    z_i    = (hidden_i . W^T + b) / T_i                      scaled logits
    lse_i  = log sum_v exp(z_iv)
    logp_i = z_i[t_i] - lse_i        if 0 <= t_i < V, else exactly 0.0

and the first-order backward for an upstream gradient g_i on logp_i:

    dz_iv      = G_i * (onehot(t_i)_v - exp(z_iv - lse_i)) / T_i,
                 G_i = g_i if t_i is in range else 0
    d_hidden   = dz @ W
    d_W        = dz^T @ hidden
    d_bias     = sum_i dz_i

Sources (the pages this follows):
  * "Fused Linear LogP" docs page, section "Reference Semantics": the linear
    layer, log_softmax over the vocabulary and the gather at the target;
    section "Tensor Contract": output z[target] - logsumexp(z), float32
    output, bias optional and differentiable; intro: gradients flow into
    hidden, lm_head_weight and bias.
  * "Feat/nemotron h lm head logprob cuda" (PR #555), summary bullets: the
    optional per-row temperature and the deterministic dlogits backward.
  * "[FEAT][kernels]: add backward support for fused logp CUDA kernels"
    (PR #234), section "Implementation details": the dlogits expression
    grad_out * (one_hot(token) - softmax(logits)); its inline review: labels
    below zero or at least the vocabulary size give the 0 result.
  * PR #547 page (deterministic LogP autograd), section "What", "Indexed
    semantics": out-of-range tokens are ignored and have zero derivatives;
    the indexed variants keep the full row shape, select a duplicated row id
    once, ignore out-of-range ids and give unselected rows zero derivatives.

Readings where the pages leave a step open (also listed with the rest of the
design notes):
  * The temperature divides the logits before the softmax: z = (hW^T + b)/T.
    Hence lse is the log-sum-exp of the scaled logits and every gradient
    carries the factor 1/T.  T is not differentiated.
  * An out-of-range target (t < 0 or t >= V, compared in int64, no wrap)
    gives logp = 0.0 exactly and contributes nothing to any gradient; the lse
    of such a row is still its true, finite log-sum-exp.
  * The bias is added before the temperature division.

Every function here is pinned by the CPU test suite to closed forms,
invariants, library routines and finite differences.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "as_f64",
    "logits",
    "row_lse",
    "valid_mask",
    "select_logp",
    "dlogits",
    "forward",
    "backward",
    "logits_forward",
    "logits_backward",
    "selected_rows",
    "forward_indexed",
    "backward_indexed",
    "logits_forward_indexed",
    "logits_backward_indexed",
    "embedding_forward",
    "embedding_backward",
]


def as_f64(x):
    """Exact up-cast of a numpy array or a CPU/GPU torch tensor to float64."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # a torch tensor: .double() is exact for bf16/fp32
        return x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def _as_i64(t):
    if hasattr(t, "detach"):
        return t.detach().to("cpu").long().numpy()
    return np.asarray(t, dtype=np.int64)


def logits(H, W, bias=None, temperature=None):
    """Scaled logits z = (H W^T + b) / T for a block of rows.

    "Fused Linear LogP", section "Reference Semantics" (linear layer with an
    optional bias); the per-row temperature of PR #555's summary divides the
    biased logits of its row.
    """
    Z = H @ W.T
    if bias is not None:
        Z = Z + bias[None, :]
    if temperature is not None:
        Z = Z / temperature[:, None]
    return Z


def row_lse(Z):
    """Per-row log-sum-exp over the vocabulary, with the row max taken out.

    "Fused Linear LogP", section "Tensor Contract": the logsumexp(z) term.
    """
    m = Z.max(axis=1)
    return m + np.log(np.exp(Z - m[:, None]).sum(axis=1))


def valid_mask(t, V):
    """In-range targets: 0 <= t < V, compared in int64 (no wrap-around).

    PR #234 inline review (labels below zero or at least the vocabulary size
    give the 0 result) and PR #547 "What" (out-of-range ids are ignored).
    """
    t = _as_i64(t)
    return (t >= 0) & (t < V)


def select_logp(Z, lse, t):
    """logp_i = z_i[t_i] - lse_i for in-range targets, exactly 0.0 otherwise.

    "Fused Linear LogP", "Tensor Contract": z[target] - logsumexp(z).
    """
    t = _as_i64(t)
    V = Z.shape[1]
    ok = valid_mask(t, V)
    safe_t = np.where(ok, t, 0)
    zt = Z[np.arange(Z.shape[0]), safe_t]
    return np.where(ok, zt - lse, 0.0)


def dlogits(Z, lse, t, g, temperature=None):
    """Gradient of sum_i g_i logp_i with respect to the *unscaled* logits.

    PR #234 "Implementation details": g * (one_hot(token) - softmax(z)); the
    chain rule through z = u / T multiplies by 1/T.  Rows with an
    out-of-range target have zero derivative (PR #547 "What").
    """
    t = _as_i64(t)
    n, V = Z.shape
    ok = valid_mask(t, V)
    G = np.where(ok, np.asarray(g, dtype=np.float64), 0.0)
    if temperature is not None:
        G = G / temperature
    P = np.exp(Z - lse[:, None])
    dZ = -G[:, None] * P
    rows = np.nonzero(ok)[0]
    dZ[rows, t[rows]] += G[rows]
    return dZ


def forward(hidden, weight, targets, bias=None, temperature=None, rows=None, chunk=512):
    """Oracle forward.  Returns (logp, lse) as float64 arrays.

    ``rows`` restricts the computation to a subset of row indices (every
    output row depends on its own row only), which is how the tests sample
    full-size launches.  Rows are processed ``chunk`` at a time.
    """
    H = as_f64(hidden)
    W = as_f64(weight)
    b = as_f64(bias)
    T = as_f64(temperature)
    t = _as_i64(targets)
    idx = np.arange(H.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    logp = np.zeros(idx.shape[0])
    lse = np.zeros(idx.shape[0])
    for s in range(0, idx.shape[0], chunk):
        r = idx[s:s + chunk]
        Z = logits(H[r], W, b, None if T is None else T[r])
        l = row_lse(Z)
        lse[s:s + chunk] = l
        logp[s:s + chunk] = select_logp(Z, l, t[r])
    return logp, lse


def backward(hidden, weight, targets, grad_out, bias=None, temperature=None, rows=None,
             chunk=512, need_weight=True, need_bias=True):
    """Oracle backward.  Returns (d_hidden, d_weight, d_bias) in float64.

    d_hidden has one row per requested row.  d_weight / d_bias sum over the
    requested rows only: they equal the full gradients when grad_out is zero
    on every other row.
    """
    H = as_f64(hidden)
    W = as_f64(weight)
    b = as_f64(bias)
    T = as_f64(temperature)
    g = as_f64(grad_out)
    t = _as_i64(targets)
    idx = np.arange(H.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    V, D = W.shape
    d_hidden = np.zeros((idx.shape[0], D))
    d_weight = np.zeros((V, D)) if need_weight else None
    d_bias = np.zeros(V) if need_bias else None
    for s in range(0, idx.shape[0], chunk):
        r = idx[s:s + chunk]
        Tr = None if T is None else T[r]
        Z = logits(H[r], W, b, Tr)
        l = row_lse(Z)
        dZ = dlogits(Z, l, t[r], g[r], Tr)
        d_hidden[s:s + chunk] = dZ @ W
        if need_weight:
            d_weight += dZ.T @ H[r]
        if need_bias:
            d_bias += dZ.sum(axis=0)
    return d_hidden, d_weight, d_bias


# ---- the sibling operator on materialised logits ---------------------------------------------
#
# "Fused LogP" (the docs page's intro contrasts it with the linear op: it takes
# already-materialised logits), with PR #547's and PR #234's conventions: the
# same lse / selected log-probability / dlogits definitions applied to given
# logits, no projection, no bias, no temperature.

def logits_forward(logits_in, targets, rows=None, chunk=512):
    """(logp, lse) of given logits [N, V], float64, exactly up-cast.

    PR #234 "Summary" (fused logp over logits) with the Tensor Contract's
    z[target] - logsumexp(z); out-of-range targets give 0.0 (PR #547 "What").
    """
    Z = as_f64(logits_in)
    t = _as_i64(targets)
    idx = np.arange(Z.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    logp = np.zeros(idx.shape[0])
    lse = np.zeros(idx.shape[0])
    for s in range(0, idx.shape[0], chunk):
        r = idx[s:s + chunk]
        l = row_lse(Z[r])
        lse[s:s + chunk] = l
        logp[s:s + chunk] = select_logp(Z[r], l, t[r])
    return logp, lse


def logits_backward(logits_in, targets, grad_out, rows=None, chunk=512):
    """d logits of sum_i g_i logp_i, float64 [rows, V] (PR #234 "Implementation
    details": g * (one_hot(token) - softmax(logits))), recomputing lse."""
    Z = as_f64(logits_in)
    t = _as_i64(targets)
    g = as_f64(grad_out)
    idx = np.arange(Z.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((idx.shape[0], Z.shape[1]))
    for s in range(0, idx.shape[0], chunk):
        r = idx[s:s + chunk]
        l = row_lse(Z[r])
        out[s:s + chunk] = dlogits(Z[r], l, t[r], g[r])
    return out


# ---- indexed (row-subset) variants ------------------------------------------------------------
#
# PR #547 page, section "What", indexed semantics: the outputs keep the full row
# shape; an id listed more than once selects its row once; an id outside the
# batch is ignored; rows that are not selected have zero derivatives.  PR #234,
# "Implementation details": rows left out by an indexed call get exactly zero
# gradients.  Reading adopted for the forward outputs of rows left out: logp and
# lse are 0 (the allocating variant's zero-filled output).

def selected_rows(n_rows_total, ids):
    """The rows an id list selects: the distinct ids in [0, n_rows_total), ascending."""
    r = _as_i64(ids).reshape(-1)
    r = r[(r >= 0) & (r < n_rows_total)]
    return np.unique(r)


def forward_indexed(hidden, weight, targets, ids, bias=None, temperature=None, chunk=512):
    """(logp, lse) [N] float64: the dense oracle on the selected rows, 0 elsewhere."""
    N = int(hidden.shape[0])
    s = selected_rows(N, ids)
    logp, lse = np.zeros(N), np.zeros(N)
    if s.size:
        logp[s], lse[s] = forward(hidden, weight, targets, bias, temperature, rows=s, chunk=chunk)
    return logp, lse


def backward_indexed(hidden, weight, targets, grad_out, ids, bias=None, temperature=None,
                     chunk=512):
    """(d_hidden [N, D], d_weight [V, D], d_bias [V]) float64: the dense oracle on the selected
    rows; d_hidden rows left out are 0, d_weight and d_bias sum over the selected rows."""
    N, D = int(hidden.shape[0]), int(hidden.shape[1])
    V = int(weight.shape[0])
    s = selected_rows(N, ids)
    d_hidden, d_weight, d_bias = np.zeros((N, D)), np.zeros((V, D)), np.zeros(V)
    if s.size:
        d_hidden[s], d_weight, d_bias = backward(hidden, weight, targets, grad_out, bias,
                                                 temperature, rows=s, chunk=chunk)
    return d_hidden, d_weight, d_bias


def logits_forward_indexed(logits_in, targets, ids, chunk=512):
    """(logp, lse) [N] float64 of given logits on the selected rows, 0 elsewhere."""
    N = int(logits_in.shape[0])
    s = selected_rows(N, ids)
    logp, lse = np.zeros(N), np.zeros(N)
    if s.size:
        logp[s], lse[s] = logits_forward(logits_in, targets, rows=s, chunk=chunk)
    return logp, lse


def logits_backward_indexed(logits_in, targets, grad_out, ids, chunk=512):
    """d logits [N, V] float64 on the selected rows, zero rows elsewhere."""
    N, V = int(logits_in.shape[0]), int(logits_in.shape[1])
    s = selected_rows(N, ids)
    out = np.zeros((N, V))
    if s.size:
        out[s] = logits_backward(logits_in, targets, grad_out, rows=s, chunk=chunk)
    return out


# ---- untied embedding lookup --------------------------------------------------------------------
#
# "Feat/nemotron h lm head logprob cuda" (PR #555), summary bullets: the untied
# embedding lookup of the same model row, with a sorted-segment grad_weight.
# The plain definitions: the lookup copies row ids[i] of the table; the
# gradient of sum_i <grad_i, E[ids_i]> with respect to row v of E is the sum of
# grad_i over the tokens with ids_i == v.  Reading adopted: an id outside
# [0, V) reads as a zero row and contributes nothing (the path's convention for
# out-of-range ids).

def embedding_forward(weight, ids):
    """[N, D] float64: row ids[i] of weight, a zero row for ids outside [0, V)."""
    E = as_f64(weight)
    i = _as_i64(ids).reshape(-1)
    ok = (i >= 0) & (i < E.shape[0])
    out = np.zeros((i.shape[0], E.shape[1]))
    out[ok] = E[i[ok]]
    return out


def embedding_backward(grad, ids, num_embeddings):
    """[V, D] float64: for each row v the sum of the gradient rows of the tokens with id v."""
    G = as_f64(grad).reshape(-1, as_f64(grad).shape[-1])
    i = _as_i64(ids).reshape(-1)
    ok = (i >= 0) & (i < num_embeddings)
    out = np.zeros((num_embeddings, G.shape[1]))
    np.add.at(out, i[ok], G[ok])
    return out
