"""Bitwise batch invariance and determinism of the HIP path (PR #555,
"Acceptance checks": batch sizes 1/2/7/64/255/257 on random row subsets, a
[3, 100] leading shape, repeat runs, train vs rollout entry, grad_hidden rows at
1/7/64/257; chunking of the backward is bit-neutral)."""
import numpy as np
import pytest
import torch

import flp_inputs
from gpu_common import flp, gpu_backward, gpu_forward, inputs, say, to_gpu, workspace_for_chunk

pytestmark = pytest.mark.gpu
BF16 = torch.bfloat16


@pytest.fixture(scope="module")
def rollout():
    inp = inputs("rollout_n8192")
    g = to_gpu(inp)
    logp, lse = gpu_forward(g)
    return inp, g, logp, lse


def _subset(g, rows):
    idx = torch.as_tensor(rows, device=g["hidden"].device)
    sub = dict(g)
    for k in ("hidden", "targets", "temperature", "grad_out"):
        if g.get(k) is not None:
            sub[k] = g[k][idx].contiguous()
    return sub


@pytest.mark.parametrize("n", [1, 2, 7, 64, 255, 257, 4096])
def test_forward_row_subsets(rollout, n):
    """A row's logp and lse do not depend on the other rows or on N (different N
    select different row-tile kernels)."""
    inp, g, logp, lse = rollout
    rows = flp_inputs.random_rows(8192, n, seed=1000 + n).numpy()
    rows = np.random.default_rng(n).permutation(rows)  # also scramble the order
    lp, ls = gpu_forward(_subset(g, rows))
    say(f"subset n={n}")
    assert torch.equal(lp, logp[rows]) and torch.equal(ls, lse[rows])


def test_forward_leading_shape(rollout):
    inp, g, logp, lse = rollout
    rows = flp_inputs.random_rows(8192, 300, seed=7).numpy()
    sub = _subset(g, rows)
    sub3 = {k: (v.reshape(3, 100, *v.shape[1:]) if k in ("hidden", "targets", "temperature")
                else v) for k, v in sub.items()}
    lp, ls = gpu_forward(sub3)
    assert lp.shape == (3, 100)
    assert torch.equal(lp.reshape(-1), logp[rows]) and torch.equal(ls.reshape(-1), lse[rows])


def test_forward_repeat_and_rollout_entry(rollout):
    inp, g, logp, lse = rollout
    lp2, ls2 = gpu_forward(g)
    lp3, none = gpu_forward(g, return_lse=False)
    assert none is None
    assert torch.equal(lp2, logp) and torch.equal(ls2, lse) and torch.equal(lp3, logp)


def test_int32_targets_same_bits(rollout):
    inp, g, logp, lse = rollout
    g32 = dict(g)
    g32["targets"] = g["targets"].to(torch.int32)
    lp, ls = gpu_forward(g32)
    assert torch.equal(lp, logp) and torch.equal(ls, lse)


@pytest.fixture(scope="module")
def train_small():
    inp = inputs("train_n16384", n_rows=1100)
    g = to_gpu(inp)
    logp, lse = gpu_forward(g)
    return inp, g, logp, lse


@pytest.mark.parametrize("n", [1, 7, 64, 100, 257, 700])
def test_d_hidden_row_subsets(train_small, n):
    """d_hidden of a row does not depend on the batch: the subsets take every d_hidden
    tile shape (64 x 16, 64 x 32, 128 x 64, 128 x 128) against the full batch's
    256 x 224 tiles."""
    inp, g, logp, lse = train_small
    dh, _, _ = gpu_backward(g, lse, need_weight=False, need_bias=False)
    rows = flp_inputs.random_rows(1100, n, seed=2000 + n).numpy()
    sub = _subset(g, rows)
    lp_s, lse_s = gpu_forward(sub)
    assert torch.equal(lse_s, lse[rows])
    dh_s, _, _ = gpu_backward(sub, lse_s, need_weight=False, need_bias=False)
    say(f"d_hidden subset n={n}")
    assert torch.equal(dh_s, dh[rows])


def test_backward_chunking_is_bit_neutral(train_small):
    """Several row chunks give exactly the bits of one chunk (PR #555 summary bullets:
    chunked deterministic backward).  Workspaces are sized with the library's planner so
    that the chunk counts are what the test says (a bf16 d_weight in several chunks needs
    the 1.4 GB fp32 accumulator, which at 1100 rows costs more than one whole chunk, so
    that path is compared at the long-sequence shape)."""
    inp, g, logp, lse = train_small
    m = flp()
    N, D, V = 1100, 2688, 131072
    F32 = torch.float32
    # d_hidden and d_bias: 256-row chunks (5) and 512-row chunks (3) against one chunk
    one = gpu_backward(g, lse, need_weight=False, need_bias=True)
    for rows in (256, 512):
        ws = workspace_for_chunk(N, D, V, BF16, BF16, rows, need_weight=False)
        dh, _, db = gpu_backward(g, lse, need_weight=False, need_bias=True, workspace_bytes=ws)
        say(f"chunking {rows} rows: d_hidden, d_bias")
        assert torch.equal(dh, one[0]) and torch.equal(db, one[2]), rows
    # fp32 d_weight accumulates in the caller's buffer: 256-row chunks against one chunk
    f1 = gpu_backward(g, lse, need_bias=True, dw_dtype=F32)
    ws = workspace_for_chunk(N, D, V, BF16, F32, 256)
    f2 = gpu_backward(g, lse, need_bias=True, dw_dtype=F32, workspace_bytes=ws)
    say("chunking 256 rows: fp32 d_weight")
    for a_, b_ in zip(f1, f2):
        assert torch.equal(a_, b_)
    # bf16 d_weight is the single rounding of the fp32 one
    full = gpu_backward(g, lse, need_bias=True)
    assert torch.equal(f1[1].to(BF16), full[1])
    assert torch.equal(full[0], one[0]) and torch.equal(full[2], one[2])


def test_fp16_row_subsets():
    """fp16 inputs take the same kernels with the fp16 MFMA: rows stay bitwise
    independent of the batch.  The full batch (1100 rows) runs d_hidden in 256 x 224
    tiles, the subsets in each of the small-batch tiles (64 x 16, 64 x 32, 128 x 64,
    128 x 128)."""
    w = flp_inputs.Workload("fp16_inv", 300, 1100, 512, 4096, torch.float16, w_std=0.06,
                            bias_std=0.1, n_ignored=4, ignore_values=(-1, 4096),
                            temperature=(0.5, 1.5), grad="normal", leading=(1100,))
    g = to_gpu(flp_inputs.make_inputs(w))
    logp, lse = gpu_forward(g)
    dh, _, _ = gpu_backward(g, lse, need_weight=False, need_bias=False)
    for n in (1, 7, 100, 257, 700):
        rows = flp_inputs.random_rows(1100, n, seed=300 + n).numpy()
        sub = _subset(g, rows)
        lp, ls = gpu_forward(sub)
        dhs, _, _ = gpu_backward(sub, ls, need_weight=False, need_bias=False)
        idx = torch.as_tensor(rows, device=logp.device)
        say(f"  fp16 subset n={n}")
        assert torch.equal(lp, logp[idx]) and torch.equal(ls, lse[idx])
        assert torch.equal(dhs, dh[idx])


def test_bf16_rounding_of_denormal_dweight():
    """The bf16 outputs are rounded to nearest even with denormals kept: with grad_out
    scaled to 1e-36, dz and d_weight fall in the denormal range, and the bf16 d_weight
    is still bit for bit the round-to-nearest-even of the fp32 d_weight of the same
    accumulation (the conversion done on the CPU by torch)."""
    w = flp_inputs.Workload("denormal_dw", 310, 64, 256, 4096, BF16, w_std=0.05,
                            bias_std=0.1, n_ignored=2, ignore_values=(-1,),
                            temperature=None, grad="normal", leading=(64,))
    g = to_gpu(flp_inputs.make_inputs(w))
    g["grad_out"] = g["grad_out"] * 1e-36
    say("case denormal_dw: N=64 D=256 V=4096 bf16, grad_out x 1e-36")
    _, lse = gpu_forward(g)
    _, dw16, _ = gpu_backward(g, lse, need_bias=False)
    _, dw32, _ = gpu_backward(g, lse, need_bias=False, dw_dtype=torch.float32)
    f = dw32.cpu()
    tiny = torch.finfo(torch.float32).tiny
    n_den = int(((f != 0) & (f.abs() < tiny)).sum())
    say(f"  fp32 d_weight entries in the denormal range: {n_den} of {f.numel()}")
    assert n_den > 1000
    assert torch.equal(f.to(BF16), dw16.cpu())
