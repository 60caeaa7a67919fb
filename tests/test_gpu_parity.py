"""HIP path vs the CPU FP64 oracle, element by element, through the C ABI.

Small cases (several tiles and ragged tails in every dimension) are compared on
every output.  The full-size workloads run in the launch configuration the
benchmark uses and are compared on sampled rows the oracle computes one by one;
d_weight / d_bias at full size use a grad_out that is non-zero on sampled rows
only (every other row then contributes exactly zero), plus properties that hold
at any size."""
import dataclasses
import os
import time

import numpy as np
import pytest
import torch

import flp_inputs
from gpu_common import (FP32_CELL, LOGP_CELL, REDUCTION_CELL, check_close, flp, gpu_backward,
                        workspace_for_chunk,
                        gpu_forward, inputs, oracle_backward, oracle_forward, say, to_gpu)

pytestmark = pytest.mark.gpu

BF16 = torch.bfloat16


def cells(dtype):
    return (FP32_CELL, FP32_CELL) if dtype == torch.float32 else (LOGP_CELL, REDUCTION_CELL)


def full_check(inp, g, dtype, dw_dtype=None):
    lc, rc = cells(dtype)
    logp, lse = gpu_forward(g)
    rl, rs = oracle_forward(inp)
    check_close("logp", logp, rl, **lc)
    check_close("lse", lse, rs, **lc)
    dh, dw, db = gpu_backward(g, lse, dw_dtype=dw_dtype, need_bias=True)
    odh, odw, odb = oracle_backward(inp)
    check_close("d_hidden", dh, odh, **lc)
    check_close("d_weight", dw, odw, **rc)
    check_close("d_bias", db, odb, **rc)
    # ignored rows: logp exactly 0 and a zero gradient row
    t = inp["targets"].numpy()
    ign = (t < 0) | (t >= inp["workload"].V)
    if ign.any():
        assert np.all(logp.cpu().numpy()[ign] == 0.0)
        assert np.all(dh.float().cpu().numpy()[ign] == 0.0)


def test_tiny_fp32_fwd_bwd():
    """The tiny fp32 workload (N=64, D=256, V=4096, 4 ignored rows), every output."""
    say("case tiny_fp32: N=64 D=256 V=4096 fp32")
    inp = inputs("tiny_fp32")
    full_check(inp, to_gpu(inp), torch.float32)


SMALL = [
    # (dtype, N, D, V, bias_std, temperature, t_dtype, n_ignored)
    (BF16, 300, 512, 4133, 0.1, (0.5, 1.5), torch.int32, 7),
    (BF16, 77, 96, 1000, None, (0.7, 1.3), torch.int64, 3),
    (torch.float32, 300, 96, 4133, 0.1, None, torch.int64, 5),
    (BF16, 513, 2688, 2048, 0.1, (0.5, 1.5), torch.int64, 9),
    (BF16, 1, 64, 300, None, None, torch.int64, 0),
    # fp16 inputs (the docs page's Tensor Contract: bf16 / fp16 / fp32)
    (torch.float16, 300, 512, 4133, 0.1, (0.5, 1.5), torch.int64, 7),
    (torch.float16, 513, 2688, 2048, 0.1, None, torch.int32, 9),
    # fp16 through each small-batch d_hidden tile: 64 x 16 (<= 64 rows), 64 x 32
    # (<= 128), 128 x 64 (<= 512, the 300-row case above), 128 x 128 (<= 1024)
    (torch.float16, 40, 320, 3000, 0.1, (0.5, 1.5), torch.int64, 3),
    (torch.float16, 100, 320, 3000, None, None, torch.int32, 4),
    (torch.float16, 700, 320, 1300, 0.1, (0.5, 1.5), torch.int64, 6),
    # an odd number of 128-byte K stages (D = 192: three), so that the last stage's
    # fragments come from LDS buffer 0, the one the forward epilogue reuses
    (BF16, 200, 192, 1500, 0.1, (0.5, 1.5), torch.int64, 3),
    # d_hidden column tiles only partly inside D: 128 x 64 tiles over D = 96 and
    # 128 x 128 tiles over D = 160
    (BF16, 150, 96, 1000, 0.1, (0.5, 1.5), torch.int64, 3),
    (BF16, 600, 160, 777, None, None, torch.int64, 4),
    # at most 32 rows over at most 256 vocabulary tiles: the forward's four-stage ring,
    # with an odd number of 64-byte K steps (D = 96: two stages, fewer than the ring;
    # D = 2080: 33 stages, the last one half)
    (BF16, 30, 96, 5000, 0.1, (0.5, 1.5), torch.int64, 2),
    (BF16, 24, 2080, 3000, None, None, torch.int32, 2),
    # the smallest shapes the gates allow: D = 32 (a single half K stage), V = 1
    (BF16, 50, 32, 700, 0.1, None, torch.int64, 2),
    (BF16, 33, 64, 1, 0.1, (0.5, 1.5), torch.int64, 2),
    (torch.float32, 20, 32, 1, None, None, torch.int32, 1),
]


def small_inputs(case, k):
    dtype, N, D, V, bstd, temp, tdt, nign = case
    w = flp_inputs.Workload(f"small{k}", 100 + k, N, D, V, dtype, w_std=1.0 / np.sqrt(D) * 1.3,
                            bias_std=bstd, n_ignored=nign,
                            ignore_values=(-1, V, -7, V + 3), temperature=temp,
                            grad="normal", leading=(N,))
    inp = flp_inputs.make_inputs(w)
    inp["targets"] = inp["targets"].to(tdt)
    return inp


@pytest.mark.parametrize("k", range(len(SMALL)))
def test_small_ragged(k):
    case = SMALL[k]
    say(f"case small{k}: {case}")
    inp = small_inputs(case, k)
    full_check(inp, to_gpu(inp), case[0])


@pytest.mark.parametrize("V", [60000, 140000])
def test_merge_shapes_and_leaves(V):
    """The slab merge's leaf paths through both of its workgroup shapes: V = 60000 has
    235 vocabulary tiles, one per leaf (tile partials held in registers); V = 140000
    has 547, three per leaf (the general path, which reads the partials twice).
    2100 rows (eight rows per workgroup) and a 40-row subset (one row per workgroup)
    match the oracle and give every row the same bits."""
    case = (BF16, 2100, 64, V, 0.1, (0.5, 1.5), torch.int64, 5)
    say(f"case merge_shapes: {case}")
    inp = small_inputs(case, 90)
    g = to_gpu(inp)
    logp, lse = gpu_forward(g)
    rl, rs = oracle_forward(inp)
    check_close("logp", logp, rl, **LOGP_CELL)
    check_close("lse", lse, rs, **LOGP_CELL)
    idx = flp_inputs.random_rows(2100, 40, seed=5).to(g["hidden"].device)
    sub = dict(g)
    for k in ("hidden", "targets", "temperature"):
        sub[k] = g[k][idx].contiguous()
    lp, ls = gpu_forward(sub)
    assert torch.equal(lp, logp[idx]) and torch.equal(ls, lse[idx])


@pytest.mark.parametrize("dtype", [BF16, torch.float32])
def test_targets_at_tile_edges(dtype):
    """Targets placed where the logit-tile epilogues branch: every row's target in
    the last, ragged vocabulary tile (on the last real column, the first column of
    a tile or of a wave's half, or a column near them), rows whose target sits in
    the other half of a tile, and ignored rows mixed in, with bias and
    temperature."""
    N, D, V = 260, 256, 1000  # V = 3 * 256 + 232: the last tile has 232 real columns
    w = flp_inputs.Workload("edges", 77, N, D, V, dtype, w_std=1.0 / np.sqrt(D) * 1.3,
                            bias_std=0.1, n_ignored=0, ignore_values=(-1,),
                            temperature=(0.5, 1.5), grad="normal", leading=(N,))
    inp = flp_inputs.make_inputs(w)
    picks = np.array([V - 1, 768, 896, 767, 895, 999 - 100, 0, 128, 255, 256, V - 2, -1, V, 900])
    t = picks[np.arange(N) % len(picks)]
    inp["targets"] = torch.from_numpy(t.astype(np.int64))
    say(f"case edges: N={N} D={D} V={V} {dtype}, targets cycling through {picks.tolist()}")
    full_check(inp, to_gpu(inp), dtype)


def test_small_bf16_fp32_dweight():
    """bf16 inputs with an fp32 d_weight output (one rounding less)."""
    inp = small_inputs(SMALL[0], 0)
    say("case small0 with fp32 d_weight")
    full_check(inp, to_gpu(inp), BF16, dw_dtype=torch.float32)


def test_decode_n32_full():
    """Decode-scale forward at its full size: all 32 rows against the oracle."""
    say("case decode_n32: N=32 D=2688 V=131072 bf16, forward")
    inp = inputs("decode_n32")
    g = to_gpu(inp)
    logp, lse = gpu_forward(g)
    rl, rs = oracle_forward(inp)
    check_close("logp", logp.reshape(-1), rl, **LOGP_CELL)
    check_close("lse", lse.reshape(-1), rs, **LOGP_CELL)


def test_rollout_n8192_sampled():
    """Rollout-scale forward with temperature: 48 sampled rows of the full launch."""
    say("case rollout_n8192: N=8192 D=2688 V=131072 bf16 + temperature, forward")
    inp = inputs("rollout_n8192")
    g = to_gpu(inp)
    logp, lse = gpu_forward(g)
    rows = flp_inputs.random_rows(8192, 48, seed=31).numpy()
    rl, rs = oracle_forward(inp, rows=rows)
    check_close("logp[rows]", logp.reshape(-1)[rows], rl, **LOGP_CELL)
    check_close("lse[rows]", lse.reshape(-1)[rows], rs, **LOGP_CELL)


def _sparse_grad(inp, rows):
    go = torch.zeros_like(inp["grad_out"])
    go[rows] = inp["grad_out"][rows]
    return go


def _train_like(name, n_sample, ws_bytes=None):
    inp = inputs(name)
    g = to_gpu(inp)
    N = inp["workload"].N
    logp, lse = gpu_forward(g)
    rows = flp_inputs.random_rows(N, n_sample, seed=41).numpy()
    rl, rs = oracle_forward(inp, rows=rows)
    check_close("logp[rows]", logp[rows], rl, **LOGP_CELL)
    check_close("lse[rows]", lse[rows], rs, **LOGP_CELL)
    t = inp["targets"].numpy()
    ign = (t < 0) | (t >= inp["workload"].V)
    assert np.all(logp.cpu().numpy()[ign] == 0.0)

    # dense grad_out: d_hidden rows are per-row, so the oracle computes the sampled ones
    dh, dw, db = gpu_backward(g, lse, need_bias=True, workspace_bytes=ws_bytes)
    odh, _, _ = oracle_backward(inp, rows=rows, need_weight=False, need_bias=False)
    check_close("d_hidden[rows]", dh[rows], odh, **LOGP_CELL)
    assert np.all(dh.float().cpu().numpy()[ign] == 0.0)
    # Every valid row's dlogits sums to zero over the vocabulary, up to the fp32
    # rounding of its lse: sum_v exp(z - lse^) = exp(lse - lse^) with
    # |lse - lse^| <= (|lse| + 1) 2^-21 (a few roundings of the sum, the log and
    # the add), which is below 1e-5 at these logit scales; the errors of a row
    # share one sign, so the bound adds them over rows.
    G = np.abs(inp["grad_out"].numpy())
    G[ign] = 0.0
    bound = 1e-5 * float(G.sum()) + 1e-3
    tot = float(db.double().sum())
    say(f"  sum_v d_bias = {tot:.3e} (bound {bound:.3e})")
    assert abs(tot) < bound
    # bitwise determinism: a second run
    dh2, dw2, db2 = gpu_backward(g, lse, need_bias=True, workspace_bytes=ws_bytes)
    assert torch.equal(dh, dh2) and torch.equal(dw, dw2) and torch.equal(db, db2)
    del dh2, dw2, db2

    # sparse grad_out: the oracle's d_weight / d_bias over the sampled rows are the full answer
    go = _sparse_grad(inp, rows)
    sdh, sdw, sdb = gpu_backward(g, lse, grad_out=go.to(g["hidden"].device), need_bias=True,
                                 workspace_bytes=ws_bytes)
    odh, odw, odb = oracle_backward(inp, grad_out=go, rows=rows)
    check_close("sparse d_weight", sdw, odw, **REDUCTION_CELL)
    check_close("sparse d_bias", sdb, odb, **REDUCTION_CELL)
    check_close("sparse d_hidden[rows]", sdh[rows], odh, **LOGP_CELL)
    others = np.setdiff1d(np.arange(N), rows)
    assert torch.count_nonzero(sdh[torch.as_tensor(others, device=sdh.device)]) == 0


def test_train_n16384():
    say("case train_n16384: N=16384 D=2688 V=131072 bf16, bias, fwd+bwd")
    _train_like("train_n16384", 32)


@pytest.mark.timeout(900)
def test_train_n16384_dense_grad_every_element():
    """The training workload with its own dense grad_out ~ N(0, 1): every element of
    d_weight and d_bias (reduction cell) and of d_hidden, logp and lse (log-prob cell)
    against the oracle over all 16384 rows, so that the error accumulated over 16384
    real contributions to each d_weight / d_bias entry is measured (PR #555,
    "det-GEMM split verification" and "Tolerance").  The oracle takes about a minute
    on 16 host cores."""
    say("case train_n16384 dense grad: N=16384 D=2688 V=131072 bf16, bias, every element")
    inp = inputs("train_n16384")
    g = to_gpu(inp)
    logp, lse = gpu_forward(g)
    dh, dw, db = gpu_backward(g, lse, need_bias=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    rl, rs = oracle_forward(inp)
    t1 = time.perf_counter()
    check_close("logp", logp, rl, **LOGP_CELL)
    check_close("lse", lse, rs, **LOGP_CELL)
    del rl, rs
    t2 = time.perf_counter()
    odh, odw, odb = oracle_backward(inp)
    t3 = time.perf_counter()
    say(f"  oracle over all 16384 rows: forward {t1 - t0:.1f} s, backward {t3 - t2:.1f} s "
        f"({len(os.sched_getaffinity(0))} host cores available)")
    check_close("d_hidden", dh, odh, **LOGP_CELL)
    del odh, dh
    check_close("d_bias", db, odb, **REDUCTION_CELL)
    # d_weight: 352 M entries, compared in blocks of vocabulary rows
    worst = 0.0
    for v0 in range(0, odw.shape[0], 16384):
        blk = slice(v0, v0 + 16384)
        worst = max(worst, check_close(f"d_weight[{v0}:{v0 + 16384}]", dw[blk], odw[blk],
                                       **REDUCTION_CELL))
    say(f"  d_weight over all rows: max|err| = {worst:.3e}")


def test_longseq_n65600_multichunk():
    """N=65600 with 5% out-of-range targets, backward in several row chunks (the
    fp32 d_weight accumulator path)."""
    say("case longseq_n65600: N=65600 D=2688 V=131072 bf16, fwd+bwd, 16384-row chunks")
    m = flp()
    ws = m.backward_workspace_bytes(65600, 2688, 131072, BF16, chunk_rows=16384)
    assert m.flp_backward_chunk_rows(65600, 2688, 131072, m.FLP_BF16, m.FLP_BF16, ws) == 16384
    _train_like("longseq_n65600", 24, ws_bytes=ws)


def test_longseq_chunked_equals_one_chunk():
    """The long sequence's backward in five row chunks (bf16 d_weight through the fp32
    accumulator across chunks) against one chunk of all 65600 rows (a 33 GiB workspace):
    every output bit for bit (PR #555 summary bullets: chunking of the deterministic
    backward is bit-neutral)."""
    m = flp()
    inp = inputs("longseq_n65600")
    g = to_gpu(inp)
    logp, lse = gpu_forward(g)
    ws5 = m.backward_workspace_bytes(65600, 2688, 131072, BF16, chunk_rows=16384)
    ws1 = workspace_for_chunk(65600, 2688, 131072, BF16, BF16, 65792, need_bias=False)
    say(f"case longseq: 5 chunks ({ws5 / 2**30:.1f} GiB) vs one chunk ({ws1 / 2**30:.1f} GiB)")
    five = gpu_backward(g, lse, need_bias=False, workspace_bytes=ws5)
    torch.cuda.synchronize()
    one = gpu_backward(g, lse, need_bias=False, workspace_bytes=ws1)
    torch.cuda.synchronize()
    assert torch.equal(five[0], one[0]), "d_hidden"
    assert torch.equal(five[1], one[1]), "d_weight"
