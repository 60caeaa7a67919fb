"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each ``pin_*`` takes the oracle module and raises (AssertionError or any
exception) when the oracle disagrees with a closed form, an invariant, a
library routine, a finite-difference derivative or the hand-worked fixture.
test_oracle.py runs them on the real oracle; test_oracle_mutants.py plants
mistakes in the oracle and checks that at least one pin catches each.
"""
from __future__ import annotations

import math
import os
import re

import numpy as np
import scipy.special
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example_3x2x3.txt")


def _rng(seed):
    return np.random.default_rng(seed)


def _case(seed, N=6, D=7, V=9, bias=True, temp=True):
    r = _rng(seed)
    H = r.standard_normal((N, D))
    W = r.standard_normal((V, D)) * 0.7
    b = r.standard_normal(V) * 0.3 if bias else None
    T = r.uniform(0.5, 1.5, N) if temp else None
    t = r.integers(0, V, N)
    return H, W, b, T, t


# ---- forward: closed forms ---------------------------------------------------------------

def pin_zero_weight_closed_form(o):
    """W = 0 and b = 0 give lse = log V and logp = -log V for every valid target, any T."""
    r = _rng(1)
    N, D, V = 7, 5, 13
    H = r.standard_normal((N, D))
    t = r.integers(0, V, N)
    T = r.uniform(0.5, 1.5, N)
    logp, lse = o.forward(H, np.zeros((V, D)), t, bias=np.zeros(V), temperature=T)
    assert np.max(np.abs(lse - math.log(V))) < 1e-14
    assert np.max(np.abs(logp + math.log(V))) < 1e-14


def pin_single_class(o):
    """V = 1: the only class has probability one, so logp = 0 and lse = z."""
    r = _rng(2)
    H = r.standard_normal((4, 3))
    W = r.standard_normal((1, 3))
    logp, lse = o.forward(H, W, np.zeros(4, dtype=np.int64))
    assert np.max(np.abs(logp)) < 1e-15
    assert np.max(np.abs(lse - (H @ W.T)[:, 0])) < 1e-14


def pin_identity_weight_log_softmax(o):
    """D = V and W = I reduce to log_softmax((h + b) / T)[t] (scipy's routine)."""
    r = _rng(3)
    N, V = 8, 11
    H = r.standard_normal((N, V)) * 2.0
    b = r.standard_normal(V)
    T = r.uniform(0.5, 1.5, N)
    t = r.integers(0, V, N)
    logp, lse = o.forward(H, np.eye(V), t, bias=b, temperature=T)
    ref = scipy.special.log_softmax((H + b) / T[:, None], axis=1)
    assert np.max(np.abs(logp - ref[np.arange(N), t])) < 1e-12
    assert np.max(np.abs(lse - scipy.special.logsumexp((H + b) / T[:, None], axis=1))) < 1e-12


def pin_cross_entropy_library(o):
    """General W (non-symmetric, D == V and D != V): logp = -cross_entropy(z, t), torch f64."""
    for seed, (N, D, V) in ((4, (9, 12, 12)), (5, (10, 6, 17))):
        H, W, b, T, t = _case(seed, N, D, V)
        logp, lse = o.forward(H, W, t, bias=b, temperature=T)
        z = torch.nn.functional.linear(torch.from_numpy(H), torch.from_numpy(W), torch.from_numpy(b))
        z = z / torch.from_numpy(T)[:, None]
        ce = torch.nn.functional.cross_entropy(z, torch.from_numpy(t), reduction="none").numpy()
        assert np.max(np.abs(logp + ce)) < 1e-12
        assert np.max(np.abs(lse - torch.logsumexp(z, dim=1).numpy())) < 1e-12


def pin_normalisation(o):
    """sum_v exp(logp(h, t = v)) = 1: one row replicated V times with targets 0..V-1."""
    r = _rng(6)
    D, V = 5, 23
    h = r.standard_normal((1, D))
    W = r.standard_normal((V, D))
    b = r.standard_normal(V)
    T = np.full(V, 0.8)
    logp, lse = o.forward(np.repeat(h, V, axis=0), W, np.arange(V), bias=b, temperature=T)
    assert abs(np.exp(logp).sum() - 1.0) < 1e-12
    assert np.all(lse == lse[0])


def pin_bias_shift(o):
    """b + c leaves logp unchanged and shifts lse by c / T."""
    H, W, b, T, t = _case(7)
    c = 3.25
    lp0, l0 = o.forward(H, W, t, bias=b, temperature=T)
    lp1, l1 = o.forward(H, W, t, bias=b + c, temperature=T)
    assert np.max(np.abs(lp1 - lp0)) < 1e-12
    assert np.max(np.abs(l1 - l0 - c / T)) < 1e-12


def pin_weight_shift(o):
    """Adding one vector u to every row of W shifts each row's logits uniformly: logp unchanged."""
    H, W, b, T, t = _case(8)
    u = _rng(9).standard_normal(W.shape[1])
    lp0, l0 = o.forward(H, W, t, bias=b, temperature=T)
    lp1, l1 = o.forward(H, W + u[None, :], t, bias=b, temperature=T)
    assert np.max(np.abs(lp1 - lp0)) < 1e-12
    assert np.max(np.abs(l1 - l0 - (H @ u) / T)) < 1e-12


def pin_temperature_power_of_two(o):
    """T = 2^k is the same as scaling W and b by 2^-k with T = 1, bit for bit in f64."""
    H, W, b, _, t = _case(10, temp=False)
    k = np.array([-2, -1, 0, 1, 2, 3])
    T = np.ldexp(1.0, k)
    lp0, l0 = o.forward(H, W, t, bias=b, temperature=T)
    for i in range(H.shape[0]):
        s = math.ldexp(1.0, -int(k[i]))
        lp1, l1 = o.forward(H[i:i + 1], W * s, t[i:i + 1], bias=b * s)
        assert np.max(np.abs(lp1[0] - lp0[i])) < 1e-13
        assert np.max(np.abs(l1[0] - l0[i])) < 1e-13


def pin_ignored_rows(o):
    """Out-of-range targets give logp exactly 0.0, the same lse, and zero derivatives."""
    H, W, b, T, t = _case(11, N=8)
    V = W.shape[0]
    bad = np.array(t)
    bad[[1, 3, 4, 6, 7]] = [-1, -100, V, V + 12345, -(2 ** 40)]
    g = _rng(12).standard_normal(len(t))
    lp0, l0 = o.forward(H, W, t, bias=b, temperature=T)
    lp1, l1 = o.forward(H, W, bad, bias=b, temperature=T)
    ign = np.array([1, 3, 4, 6, 7])
    keep = np.array([0, 2, 5])
    assert np.all(lp1[ign] == 0.0)
    assert np.all(l1 == l0)
    assert np.all(lp1[keep] == lp0[keep])
    dh, dw, db = o.backward(H, W, bad, g, bias=b, temperature=T)
    assert np.all(dh[ign] == 0.0)
    g0 = g.copy()
    g0[ign] = 0.0
    dh0, dw0, db0 = o.backward(H, W, t, g0, bias=b, temperature=T)
    assert np.max(np.abs(dw - dw0)) < 1e-14 and np.max(np.abs(db - db0)) < 1e-14


# ---- backward -----------------------------------------------------------------------------

def _loss(o, H, W, b, T, t, g):
    lp, _ = o.forward(H, W, t, bias=b, temperature=T)
    return float(np.dot(g, lp))


def pin_finite_differences(o):
    """Central finite differences (step 1e-6, f64) of L = sum_i g_i logp_i on N=5, D=8, V=11."""
    H, W, b, T, t = _case(13, N=5, D=8, V=11)
    t = np.array(t)
    t[2] = -1
    g = _rng(14).standard_normal(5)
    dh, dw, db = o.backward(H, W, t, g, bias=b, temperature=T)
    eps = 1e-6

    def fd(arr, which):
        out = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            p = arr.copy(); p[idx] += eps
            m = arr.copy(); m[idx] -= eps
            args = {"H": H, "W": W, "b": b}
            args[which] = p
            lp = _loss(o, args["H"], args["W"], args["b"], T, t, g)
            args[which] = m
            lm = _loss(o, args["H"], args["W"], args["b"], T, t, g)
            out[idx] = (lp - lm) / (2 * eps)
        return out

    for an, which, arr in ((dh, "H", H), (dw, "W", W), (db, "b", b)):
        num = fd(arr, which)
        rel = np.linalg.norm(num - an) / max(np.linalg.norm(an), 1e-30)
        assert rel < 1e-6, (which, rel)


def pin_autograd_library(o):
    """torch.autograd on an f64 CPU expression (linear, log_softmax, gather) agrees to 1e-12."""
    H, W, b, T, t = _case(15, N=9, D=6, V=14)
    t = np.array(t)
    t[[0, 5]] = [-3, 14]
    g = _rng(16).standard_normal(9)
    Ht = torch.tensor(H, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    bt = torch.tensor(b, requires_grad=True)
    z = torch.nn.functional.linear(Ht, Wt, bt) / torch.tensor(T)[:, None]
    ls = torch.log_softmax(z, dim=1)
    tt = torch.tensor(t)
    ok = (tt >= 0) & (tt < 14)
    sel = ls.gather(1, torch.where(ok, tt, 0)[:, None])[:, 0]
    out = torch.where(ok, sel, torch.zeros_like(sel))
    (out * torch.tensor(g)).sum().backward()
    dh, dw, db = o.backward(H, W, t, g, bias=b, temperature=T)
    lp, _ = o.forward(H, W, t, bias=b, temperature=T)
    assert np.max(np.abs(lp - out.detach().numpy())) < 1e-12
    assert np.max(np.abs(dh - Ht.grad.numpy())) < 1e-12
    assert np.max(np.abs(dw - Wt.grad.numpy())) < 1e-12
    assert np.max(np.abs(db - bt.grad.numpy())) < 1e-12


def pin_gradient_invariants(o):
    """sum_v d_bias = 0 and sum_v d_W[v, :] = 0; gradients linear in grad_out; g = 0 gives 0."""
    H, W, b, T, t = _case(17, N=7, D=5, V=10)
    r = _rng(18)
    g1, g2 = r.standard_normal(7), r.standard_normal(7)
    dh1, dw1, db1 = o.backward(H, W, t, g1, bias=b, temperature=T)
    dh2, dw2, db2 = o.backward(H, W, t, g2, bias=b, temperature=T)
    dh3, dw3, db3 = o.backward(H, W, t, 2.0 * g1 - g2, bias=b, temperature=T)
    assert abs(db1.sum()) < 1e-13
    assert np.max(np.abs(dw1.sum(axis=0))) < 1e-13
    for a1, a2, a3 in ((dh1, dh2, dh3), (dw1, dw2, dw3), (db1, db2, db3)):
        assert np.max(np.abs(a3 - (2.0 * a1 - a2))) < 1e-12
    z = o.backward(H, W, t, np.zeros(7), bias=b, temperature=T)
    assert all(np.all(a == 0.0) for a in z)


def pin_row_subsets(o):
    """Each output row depends on its own row only: the rows= sampling equals the full result."""
    H, W, b, T, t = _case(19, N=12, D=4, V=8)
    g = _rng(20).standard_normal(12)
    rows = np.array([1, 4, 5, 11])
    lp, l = o.forward(H, W, t, bias=b, temperature=T)
    lps, ls = o.forward(H, W, t, bias=b, temperature=T, rows=rows, chunk=3)
    assert np.max(np.abs(lps - lp[rows])) < 1e-14 and np.max(np.abs(ls - l[rows])) < 1e-14
    gz = np.zeros(12)
    gz[rows] = g[rows]
    dh, dw, db = o.backward(H, W, t, gz, bias=b, temperature=T, chunk=5)
    dhs, dws, dbs = o.backward(H, W, t, g, bias=b, temperature=T, rows=rows, chunk=3)
    assert np.max(np.abs(dhs - dh[rows])) < 1e-14
    assert np.max(np.abs(dws - dw)) < 1e-13 and np.max(np.abs(dbs - db)) < 1e-13


# ---- hand-worked fixture --------------------------------------------------------------------

def load_golden(path=GOLDEN):
    env = {"e": math.e, "log": math.log, "sqrt": math.sqrt, "__builtins__": {}}
    data, expect = {}, {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            m = re.match(r"expect\s+(\w+)\s*=\s*(.*)$", line)
            if m:
                expect[m.group(1)] = np.array(eval(m.group(2), env), dtype=np.float64)
                continue
            k, v = [s.strip() for s in line.split("=", 1)]
            data[k] = eval(v, env)
    return data, expect


def pin_golden_worked_example(o):
    """The hand-derived 3x2x3 example (closed forms in tests/golden)."""
    d, e = load_golden()
    H = np.array(d["hidden"], dtype=np.float64)
    W = np.array(d["weight"], dtype=np.float64)
    b = np.array(d["bias"], dtype=np.float64)
    T = np.array(d["temperature"], dtype=np.float64)
    t = np.array(d["targets"], dtype=np.int64)
    g = np.array(d["grad_out"], dtype=np.float64)
    lp, l = o.forward(H, W, t, bias=b, temperature=T)
    dh, dw, db = o.backward(H, W, t, g, bias=b, temperature=T)
    for got, key in ((l, "lse"), (lp, "logp"), (dh, "d_hidden"), (dw, "d_weight"), (db, "d_bias")):
        assert got.shape == e[key].shape, key
        assert np.max(np.abs(got - e[key])) < 1e-14, key


# ---- the operator on materialised logits -----------------------------------------------------

def pin_logits_op_library(o):
    """Given logits: logp = scipy log_softmax(z)[t] (0 for ignored rows), lse = scipy logsumexp,
    d logits = torch autograd of the f64 log_softmax-gather expression."""
    r = _rng(40)
    Z = r.standard_normal((8, 13)) * 2.0
    t = r.integers(0, 13, 8)
    t[[1, 6]] = [-1, 13]
    g = r.standard_normal(8)
    lp, ls = o.logits_forward(Z, t)
    ok = (t >= 0) & (t < 13)
    ref = scipy.special.log_softmax(Z, axis=1)[np.arange(8), np.where(ok, t, 0)]
    assert np.max(np.abs(lp - np.where(ok, ref, 0.0))) < 1e-12
    assert np.all(lp[~ok] == 0.0)
    assert np.max(np.abs(ls - scipy.special.logsumexp(Z, axis=1))) < 1e-12
    Zt = torch.tensor(Z, requires_grad=True)
    tt = torch.tensor(t)
    okt = (tt >= 0) & (tt < 13)
    sel = torch.log_softmax(Zt, dim=1).gather(1, torch.where(okt, tt, 0)[:, None])[:, 0]
    (torch.where(okt, sel, torch.zeros_like(sel)) * torch.tensor(g)).sum().backward()
    dZ = o.logits_backward(Z, t, g)
    assert np.max(np.abs(dZ - Zt.grad.numpy())) < 1e-12
    assert np.all(dZ[~ok] == 0.0)


def pin_logits_op_matches_identity_linear(o):
    """The linear op with D = V, W = I, no bias and T = 1 is the logits op on h: both oracle
    paths, each pinned separately, must agree."""
    r = _rng(41)
    H = r.standard_normal((5, 7))
    t = r.integers(0, 7, 5)
    g = r.standard_normal(5)
    lp1, ls1 = o.forward(H, np.eye(7), t)
    lp2, ls2 = o.logits_forward(H, t)
    dh, _, _ = o.backward(H, np.eye(7), t, g)
    dZ = o.logits_backward(H, t, g)
    assert np.max(np.abs(lp1 - lp2)) < 1e-14 and np.max(np.abs(ls1 - ls2)) < 1e-14
    assert np.max(np.abs(dh - dZ)) < 1e-14


def pin_logits_op_finite_differences(o):
    """Central finite differences of L = sum_i g_i logp_i with respect to each logit."""
    r = _rng(42)
    Z = r.standard_normal((3, 6))
    t = np.array([2, -1, 5])
    g = r.standard_normal(3)
    an = o.logits_backward(Z, t, g)
    num = np.zeros_like(Z)
    h = 1e-6
    for i in range(3):
        for v in range(6):
            Zp, Zm = Z.copy(), Z.copy()
            Zp[i, v] += h
            Zm[i, v] -= h
            num[i, v] = ((o.logits_forward(Zp, t)[0] * g).sum()
                         - (o.logits_forward(Zm, t)[0] * g).sum()) / (2 * h)
    assert np.linalg.norm(num - an) / np.linalg.norm(an) < 1e-6


# ---- indexed (row-subset) variants ---------------------------------------------------------

_IDS = np.array([3, -1, 3, 0, 7, 0, -6])  # selects rows {0, 3} of 5; -1 / -6 / 7 are ignored


def pin_indexed_library(o):
    """Indexed forward/backward against scipy's log_softmax and torch autograd of the loss
    sum over the selected rows {0, 3} of g_i logp_i (rows 1, 2, 4 left out: zeros)."""
    H, W, b, T, t = _case(50, N=5, D=3, V=4)
    g = _rng(51).standard_normal(5)
    sel = np.array([0, 3])
    Z = (H @ W.T + b[None, :]) / T[:, None]
    ls = scipy.special.log_softmax(Z, axis=1)
    want = np.zeros(5)
    want[sel] = ls[sel, t[sel]]
    want_lse = np.zeros(5)
    want_lse[sel] = scipy.special.logsumexp(Z[sel], axis=1)
    lp, lse = o.forward_indexed(H, W, t, _IDS, bias=b, temperature=T)
    assert np.max(np.abs(lp - want)) < 1e-12 and np.max(np.abs(lse - want_lse)) < 1e-12
    assert np.all(lp[[1, 2, 4]] == 0.0) and np.all(lse[[1, 2, 4]] == 0.0)
    Ht = torch.tensor(H, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    bt = torch.tensor(b, requires_grad=True)
    z = (Ht @ Wt.T + bt) / torch.tensor(T)[:, None]
    L = (torch.log_softmax(z, dim=1)[sel, t[sel]] * torch.tensor(g[sel])).sum()
    L.backward()
    dh, dw, db = o.backward_indexed(H, W, t, g, _IDS, bias=b, temperature=T)
    assert np.max(np.abs(dh - Ht.grad.numpy())) < 1e-12
    assert np.all(dh[[1, 2, 4]] == 0.0)
    assert np.max(np.abs(dw - Wt.grad.numpy())) < 1e-12
    assert np.max(np.abs(db - bt.grad.numpy())) < 1e-12


def pin_indexed_id_lists(o):
    """The selection is a set: any order, repeats and out-of-range ids give the same result as
    the ascending distinct ids; all ids give the dense result; no ids give zeros."""
    H, W, b, T, t = _case(52, N=6, D=4, V=5)
    g = _rng(53).standard_normal(6)
    base = o.backward_indexed(H, W, t, g, np.array([1, 4]), bias=b, temperature=T)
    for ids in ([4, 1], [4, 4, 1, 1, 4], [-1, 4, 6, 1, -7, 100]):
        got = o.backward_indexed(H, W, t, g, np.array(ids), bias=b, temperature=T)
        assert all(np.array_equal(x, y) for x, y in zip(got, base)), ids
    # all rows: the dense forward (closed form via scipy) and the dense backward
    Z = (H @ W.T + b[None, :]) / T[:, None]
    lp, _ = o.forward_indexed(H, W, t, np.arange(6)[::-1], bias=b, temperature=T)
    assert np.max(np.abs(lp - scipy.special.log_softmax(Z, axis=1)[np.arange(6), t])) < 1e-12
    # nothing selected
    lp, lse = o.forward_indexed(H, W, t, np.array([], dtype=np.int64), bias=b, temperature=T)
    dh, dw, db = o.backward_indexed(H, W, t, g, np.array([-2, 6]), bias=b, temperature=T)
    assert not lp.any() and not lse.any() and not dh.any() and not dw.any() and not db.any()


def pin_logits_indexed_library(o):
    """Indexed operator on given logits against scipy and torch autograd on the selected rows."""
    r = _rng(54)
    Z = r.standard_normal((5, 7)) * 2.0
    t = np.array([1, 6, -1, 3, 9])
    g = r.standard_normal(5)
    sel = np.array([0, 3])  # _IDS selects rows 0 and 3
    ls = scipy.special.log_softmax(Z, axis=1)
    lp, lse = o.logits_forward_indexed(Z, t, _IDS)
    want = np.zeros(5)
    want[sel] = ls[sel, t[sel]]
    assert np.max(np.abs(lp - want)) < 1e-12
    assert np.max(np.abs(lse[sel] - scipy.special.logsumexp(Z[sel], axis=1))) < 1e-12
    assert np.all(lse[[1, 2, 4]] == 0.0)
    Zt = torch.tensor(Z, requires_grad=True)
    (torch.log_softmax(Zt, dim=1)[sel, t[sel]] * torch.tensor(g[sel])).sum().backward()
    d = o.logits_backward_indexed(Z, t, g, _IDS)
    assert np.max(np.abs(d - Zt.grad.numpy())) < 1e-12
    assert np.all(d[[1, 2, 4]] == 0.0)


# ---- untied embedding lookup ------------------------------------------------------------------

def pin_embedding_library(o):
    """Lookup and its gradient against torch.nn.functional.embedding and autograd (valid ids),
    and against the one-hot matrix form dE = onehot(ids)^T @ grad (a library matmul)."""
    r = _rng(60)
    V, D = 7, 5
    E = r.standard_normal((V, D))
    ids = np.array([3, 0, 3, 6, 3, 1, 0])
    G = r.standard_normal((ids.size, D))
    Et = torch.tensor(E, requires_grad=True)
    out = torch.nn.functional.embedding(torch.tensor(ids), Et)
    (out * torch.tensor(G)).sum().backward()
    assert np.array_equal(o.embedding_forward(E, ids), out.detach().numpy())
    dE = o.embedding_backward(G, ids, V)
    assert np.max(np.abs(dE - Et.grad.numpy())) < 1e-13
    onehot = (ids[:, None] == np.arange(V)[None, :]).astype(np.float64)
    assert np.max(np.abs(dE - onehot.T @ G)) < 1e-13
    assert not dE[[2, 4, 5]].any()  # ids that do not occur


def pin_embedding_invalid_ids_and_permutation(o):
    """Ids outside [0, V) read zero rows and add nothing; permuting tokens (ids and gradient
    rows together) leaves the gradient unchanged; the rows of dE add up to the valid grads."""
    r = _rng(61)
    V, D = 6, 4
    E = r.standard_normal((V, D))
    ids = np.array([2, -1, 5, 6, 2, 0, -3, 2])
    G = r.standard_normal((ids.size, D))
    out = o.embedding_forward(E, ids)
    ok = (ids >= 0) & (ids < V)
    assert not out[~ok].any() and np.array_equal(out[ok], E[ids[ok]])
    dE = o.embedding_backward(G, ids, V)
    assert np.max(np.abs(dE - o.embedding_backward(G[ok], ids[ok], V))) < 1e-14
    assert np.max(np.abs(dE.sum(axis=0) - G[ok].sum(axis=0))) < 1e-12
    p = r.permutation(ids.size)
    assert np.max(np.abs(o.embedding_backward(G[p], ids[p], V) - dE)) < 1e-12
    assert np.max(np.abs(dE[2] - (G[0] + G[4] + G[7]))) < 1e-14


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
