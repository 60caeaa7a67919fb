"""Indexed (row-subset) variants against the FP64 oracle's indexed functions and
against the dense calls, bit for bit (PR #547 page, section "What", indexed
semantics: full output row shape, a repeated id selects its row once, ids
outside the batch are ignored, rows left out get zero results and zero
gradients; PR #234 "Implementation details": exactly zero gradients for rows
left out).  A selected row of an indexed call must carry exactly the bits the
dense call gives it; d_weight and d_bias are the sums over the selected rows."""
import numpy as np
import pytest
import torch

import flp_inputs
import oracle
from gpu_common import (FP32_CELL, LOGP_CELL, REDUCTION_CELL, check_close, flp, gpu_backward,
                        gpu_forward, inputs, say, to_gpu)

pytestmark = pytest.mark.gpu
BF16 = torch.bfloat16


def small_case(N, D, V, dtype, seed):
    w = flp_inputs.Workload(f"idx{seed}", 300 + seed, N, D, V, dtype, w_std=1.3 / np.sqrt(D),
                            bias_std=0.1, n_ignored=4, ignore_values=(-1, V, -100, V + 3),
                            temperature=(0.5, 1.5), grad="normal", leading=(N,))
    return flp_inputs.make_inputs(w)


def run_indexed(g, ids, dw_dtype=None):
    m = flp()
    lp, ls = m.forward_indexed(g["hidden"], g["weight"], g["targets"], ids, g["bias"],
                               g["temperature"])
    dh, dw, db = m.backward_indexed(g["grad_out"], ls, g["hidden"], g["weight"], g["targets"], ids,
                                    g["bias"], g["temperature"], dw_dtype=dw_dtype)
    return lp, ls, dh, dw, db


def oracle_indexed(inp, ids):
    lp, ls = oracle.forward_indexed(inp["hidden"], inp["weight"], inp["targets"], ids,
                                    inp["bias"], inp["temperature"])
    dh, dw, db = oracle.backward_indexed(inp["hidden"], inp["weight"], inp["targets"],
                                         inp["grad_out"], ids, inp["bias"], inp["temperature"])
    return lp, ls, dh, dw, db


def check_against_dense(g, ids, got):
    """Selected rows: the dense call's bits; other rows: exact zeros."""
    lp, ls, dh, _, _ = got
    N = int(g["targets"].numel())
    sel = oracle.selected_rows(N, ids)
    keep = torch.zeros(N, dtype=torch.bool)
    keep[torch.as_tensor(sel, dtype=torch.long)] = True
    keep = keep.to(lp.device)
    lp0, ls0 = gpu_forward(g)
    dh0, _, _ = gpu_backward(g, ls0, need_weight=False, need_bias=False)
    torch.cuda.synchronize()
    assert torch.equal(lp[keep], lp0[keep]) and torch.equal(ls[keep], ls0[keep])
    assert torch.equal(dh[keep], dh0[keep])
    assert not lp[~keep].any() and not ls[~keep].any() and not dh[~keep].any()


CASES = [
    # (dtype, N, D, V, n distinct ids, repeats, out-of-range ids, id dtype)
    (BF16, 300, 256, 1300, 120, 40, (-1, 300, -7, 1 << 40), torch.int64),
    (BF16, 300, 256, 1300, 300, 10, (), torch.int32),       # every row, shuffled, repeated
    (torch.float16, 77, 128, 1000, 30, 5, (77,), torch.int32),
    (torch.float32, 64, 256, 4096, 20, 3, (-1,), torch.int64),
]


@pytest.mark.parametrize("k", range(len(CASES)))
def test_indexed_linear_parity(k):
    dtype, N, D, V, n, rep, bad, idt = CASES[k]
    say(f"indexed linear case {k}: {dtype} N={N} D={D} V={V} ids {n}+{rep}+{len(bad)} {idt}")
    if idt == torch.int32:
        bad = tuple(b for b in bad if -(1 << 31) <= b < (1 << 31))
    inp = small_case(N, D, V, dtype, k)
    ids = flp_inputs.row_ids(N, n, seed=700 + k, n_dup=rep, invalid=bad, dtype=idt)
    g = to_gpu(inp)
    got = run_indexed(g, ids.cuda())
    ref = oracle_indexed(inp, ids)
    cell = FP32_CELL if dtype == torch.float32 else LOGP_CELL
    red = FP32_CELL if dtype == torch.float32 else REDUCTION_CELL
    for name, x, r, c in zip(("logp", "lse", "d_hidden", "d_weight", "d_bias"), got, ref,
                             (cell, cell, cell, red, red)):
        check_close(name, x.float(), r, **c)
    check_against_dense(g, ids, got)


def test_indexed_all_rows_equals_dense_bitwise():
    """Selecting every row (any order, repeats) reproduces the dense call bit for bit,
    d_weight and d_bias included: the compacted rows are the batch in its own order."""
    inp = small_case(520, 256, 1300, BF16, 9)
    g = to_gpu(inp)
    ids = flp_inputs.row_ids(520, 520, seed=790, n_dup=50, invalid=(-1, 520))
    got = run_indexed(g, ids.cuda())
    lp0, ls0 = gpu_forward(g)
    dense = gpu_backward(g, ls0)
    torch.cuda.synchronize()
    assert torch.equal(got[0], lp0) and torch.equal(got[1], ls0)
    for a, b in zip(got[2:], dense):
        assert torch.equal(a, b)


def test_indexed_empty_and_all_invalid():
    inp = small_case(100, 128, 700, BF16, 11)
    g = to_gpu(inp)
    for ids in (torch.empty(0, dtype=torch.int64), torch.tensor([-1, 100, 5000, -3])):
        say(f"ids {ids.tolist()}")
        lp, ls, dh, dw, db = run_indexed(g, ids.cuda())
        torch.cuda.synchronize()
        for name, x in (("logp", lp), ("lse", ls), ("d_hidden", dh), ("d_weight", dw),
                        ("d_bias", db)):
            assert not x.any(), name


def test_indexed_fp32_d_weight_and_skips():
    """fp32 d_weight, and backward calls that request only some outputs."""
    inp = small_case(200, 128, 1000, BF16, 12)
    g = to_gpu(inp)
    ids = flp_inputs.row_ids(200, 90, seed=791, n_dup=9, invalid=(-1,)).cuda()
    m = flp()
    lp, ls, dh, dw, db = run_indexed(g, ids, dw_dtype=torch.float32)
    ref = oracle_indexed(inp, ids.cpu())
    check_close("d_weight fp32", dw, ref[3], **REDUCTION_CELL)
    dh2, dw2, db2 = m.backward_indexed(g["grad_out"], ls, g["hidden"], g["weight"], g["targets"],
                                       ids, g["bias"], g["temperature"], need_hidden=False,
                                       need_weight=True, need_bias=False,
                                       dw_dtype=torch.float32)
    torch.cuda.synchronize()
    assert dh2 is None and db2 is None and torch.equal(dw2, dw)


def test_indexed_small_workspace_same_bits():
    """The minimum backward workspace (256-row chunks) gives the same bits as one chunk."""
    inp = small_case(700, 128, 1000, BF16, 13)
    g = to_gpu(inp)
    ids = flp_inputs.row_ids(700, 600, seed=792, n_dup=30).cuda()
    m = flp()
    lp, ls = m.forward_indexed(g["hidden"], g["weight"], g["targets"], ids, g["bias"],
                               g["temperature"])
    a = m.backward_indexed(g["grad_out"], ls, g["hidden"], g["weight"], g["targets"], ids,
                           g["bias"], g["temperature"])
    lo = m.flp_backward_indexed_workspace_bytes(700, 128, 1000, m.FLP_BF16, m.FLP_BF16, ids.numel(),
                                                0)
    b = m.backward_indexed(g["grad_out"], ls, g["hidden"], g["weight"], g["targets"], ids,
                           g["bias"], g["temperature"], workspace_bytes=lo)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_indexed_autograd():
    inp = small_case(96, 128, 600, BF16, 14)
    g = to_gpu(inp)
    ids = flp_inputs.row_ids(96, 40, seed=793, n_dup=6, invalid=(96,)).cuda()
    m = flp()
    h = g["hidden"].clone().requires_grad_(True)
    w = g["weight"].clone().requires_grad_(True)
    b = g["bias"].clone().requires_grad_(True)
    logp = m.linear_logp_indexed(h, w, g["targets"], ids, b, g["temperature"])
    (logp * g["grad_out"]).sum().backward()
    _, ls = m.forward_indexed(g["hidden"], g["weight"], g["targets"], ids, g["bias"],
                              g["temperature"])
    dh, dw, db = m.backward_indexed(g["grad_out"], ls, g["hidden"], g["weight"], g["targets"], ids,
                                    g["bias"], g["temperature"])
    torch.cuda.synchronize()
    assert torch.equal(h.grad, dh) and torch.equal(w.grad, dw) and torch.equal(b.grad, db)


def test_indexed_rollout_shape_sampled():
    """D = 2688, V = 131072, N = 4096 with 1500 ids (repeats and out-of-range ids): logp,
    lse and d_hidden of the selected rows equal the dense call's bits (zeros elsewhere),
    sampled rows against the oracle, and d_weight / d_bias against the dense backward with
    grad_out zeroed outside the selection (the same sums in another order)."""
    N = 4096
    inp = inputs("rollout_n8192", n_rows=N)
    g = to_gpu(inp)
    g["grad_out"] = torch.randn(N, generator=torch.Generator().manual_seed(794)).cuda()
    ids = flp_inputs.row_ids(N, 1500, seed=795, n_dup=200, invalid=(-1, N, 10 ** 9))
    say(f"rollout-shape indexed: N={N}, {ids.numel()} ids")
    got = run_indexed(g, ids.cuda())
    check_against_dense(g, ids, got)
    sel = oracle.selected_rows(N, ids)
    sample = sel[flp_inputs.random_rows(len(sel), 8, seed=796).numpy()]
    rl, rs = oracle.forward(inp["hidden"], inp["weight"], inp["targets"], inp["bias"],
                            inp["temperature"], rows=sample)
    idx = torch.as_tensor(sample, device="cuda:0")
    check_close("logp (sampled)", got[0][idx], rl, **LOGP_CELL)
    check_close("lse (sampled)", got[1][idx], rs, **LOGP_CELL)
    rdh, _, _ = oracle.backward(inp["hidden"], inp["weight"], inp["targets"],
                                g["grad_out"].cpu(), inp["bias"], inp["temperature"], rows=sample,
                                need_weight=False, need_bias=False)
    check_close("d_hidden (sampled)", got[2][idx].float(), rdh, **LOGP_CELL)
    mask = torch.zeros(N, dtype=torch.bool)
    mask[torch.as_tensor(sel)] = True
    g0 = torch.where(mask.cuda(), g["grad_out"], torch.zeros_like(g["grad_out"]))
    _, ls0 = gpu_forward(g)
    _, dw0, db0 = gpu_backward(g, ls0, grad_out=g0, need_hidden=False,
                               need_bias=g["bias"] is not None)
    pairs = [("d_weight", got[3], dw0)] + ([("d_bias", got[4], db0)] if db0 is not None else [])
    for name, a, b in pairs:  # compared on the device: [V, D] is 352M elements
        a, b = a.float(), b.float()
        err = (a - b).abs()
        bad = int((err > REDUCTION_CELL["atol"] + REDUCTION_CELL["rtol"] * b.abs()).sum())
        say(f"  {name} vs dense with masked grad_out: max|err| = {float(err.max()):.3e}, "
            f"{bad} outside the reduction cell")
        assert bad == 0


# ---- the operator on materialised logits -----------------------------------------------------

LOGIT_CASES = [
    (BF16, 300, 4136, torch.int64),
    (torch.float16, 77, 1000, torch.int32),
    (torch.float32, 64, 4100, torch.int64),
]


@pytest.mark.parametrize("k", range(len(LOGIT_CASES)))
def test_indexed_logits_parity(k):
    dtype, N, V, idt = LOGIT_CASES[k]
    say(f"indexed logits case {k}: {dtype} N={N} V={V}")
    inp = flp_inputs.make_logits_inputs(f"ilogits{k}", N, V, dtype, 80 + k, n_ignored=3,
                                        ignore_values=(-1, V), logit_std=2.0)
    ids = flp_inputs.row_ids(N, N // 3, seed=800 + k, n_dup=N // 10, invalid=(-2, N), dtype=idt)
    m = flp()
    z, t, go = inp["logits"].cuda(), inp["targets"].cuda(), inp["grad_out"].cuda()
    lp, ls = m.logits_forward_indexed(z, t, ids.cuda())
    d = m.logits_backward_indexed(go, ls, z, t, ids.cuda())
    rl, rs = oracle.logits_forward_indexed(inp["logits"], inp["targets"], ids)
    rd = oracle.logits_backward_indexed(inp["logits"], inp["targets"], inp["grad_out"], ids)
    cell = FP32_CELL if dtype == torch.float32 else LOGP_CELL
    check_close("logp", lp, rl, **cell)
    check_close("lse", ls, rs, **cell)
    check_close("d_logits", d.float(), rd, **cell)
    # selected rows carry the dense call's bits
    lp0, ls0 = m.logits_forward(z, t)
    d0 = m.logits_backward(go, ls0, z, t)
    sel = torch.as_tensor(oracle.selected_rows(N, ids), device="cuda:0")
    torch.cuda.synchronize()
    assert torch.equal(lp[sel], lp0[sel]) and torch.equal(ls[sel], ls0[sel])
    assert torch.equal(d[sel], d0[sel])


def test_indexed_logits_autograd_and_empty():
    m = flp()
    inp = flp_inputs.make_logits_inputs("ilogits_ag", 40, 520, BF16, 90, n_ignored=2)
    z = inp["logits"].cuda().requires_grad_(True)
    t, go = inp["targets"].cuda(), inp["grad_out"].cuda()
    ids = flp_inputs.row_ids(40, 15, seed=810, n_dup=4, invalid=(40,)).cuda()
    (m.logits_logp_indexed(z, t, ids) * go).sum().backward()
    _, ls = m.logits_forward_indexed(z.detach(), t, ids)
    assert torch.equal(z.grad, m.logits_backward_indexed(go, ls, z.detach(), t, ids))
    empty = torch.empty(0, dtype=torch.int64, device="cuda:0")
    lp, ls = m.logits_forward_indexed(z.detach(), t, empty)
    d = m.logits_backward_indexed(go, ls, z.detach(), t, empty)
    torch.cuda.synchronize()
    assert not lp.any() and not ls.any() and not d.any()
