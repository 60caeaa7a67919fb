"""Untied embedding lookup and its sorted-segment grad_weight ("Feat/nemotron h
lm head logprob cuda", PR #555 summary bullets; its Known issues record that the
pages' version accumulates repeated ids in BF16 and misses FP64 parity) against
the FP64 oracle (oracle.embedding_forward / embedding_backward), bitwise
reproducibility, and the autograd node."""
import pytest
import torch

import flp_inputs
import oracle
from gpu_common import FP32_CELL, REDUCTION_CELL, check_close, flp, say

pytestmark = pytest.mark.gpu
BF16 = torch.bfloat16


def run(inp, dw_dtype=None, id_dtype=torch.int64):
    m = flp()
    w = inp["weight"].cuda()
    ids = inp["ids"].to(id_dtype).cuda()
    g = inp["grad"].cuda()
    out = m.embedding_forward(w, ids)
    dw = m.embedding_backward(g, ids, int(w.shape[0]), dw_dtype=dw_dtype)
    return out, dw


CASES = [
    # (dtype, N, D, V, id draw, out-of-range ids, id dtype, d_weight dtype)
    (BF16, 3000, 64, 5000, "zipf", (-1, 5000, -7), torch.int64, None),
    (BF16, 2500, 128, 1000, "uniform", (), torch.int32, torch.float32),
    (torch.float16, 700, 96, 300, "zipf", (300,), torch.int64, None),
    (torch.float32, 900, 36, 2000, "zipf", (-2,), torch.int32, None),
    (BF16, 1500, 64, 4000, "same", (), torch.int64, None),    # one id repeated 1500 times
    (BF16, 1, 8, 3, "uniform", (), torch.int64, None),
]


@pytest.mark.parametrize("k", range(len(CASES)))
def test_embedding_parity(k):
    dtype, N, D, V, draw, bad, idt, dwt = CASES[k]
    say(f"embedding case {k}: {dtype} N={N} D={D} V={V} ids {draw} d_weight {dwt}")
    inp = flp_inputs.make_embedding_inputs(N, D, V, dtype, 40 + k, ids=draw, invalid=bad)
    out, dw = run(inp, dwt, idt)
    torch.cuda.synchronize()
    # the lookup is a copy: exact
    ref_out = oracle.embedding_forward(inp["weight"], inp["ids"])
    assert torch.equal(out.double().cpu(), torch.from_numpy(ref_out))
    ref = oracle.embedding_backward(inp["grad"], inp["ids"], V)
    cell = FP32_CELL if (dtype == torch.float32 or dwt == torch.float32) else REDUCTION_CELL
    check_close("d_weight", dw.float(), ref, **cell)
    if dwt is None and dtype != torch.float32:
        # fp32 accumulation and one rounding: within one unit in the last place of the
        # output dtype of the exact sum (a BF16-accumulated sum is not)
        refq = torch.from_numpy(ref).to(dtype).double()
        ulp = torch.from_numpy(ref).abs().clamp_min(1e-30).log2().floor().exp2()
        ulp = ulp * (2.0 ** -7 if dtype == BF16 else 2.0 ** -10)
        assert bool(((dw.double().cpu() - refq).abs() <= ulp).all())


def test_embedding_deterministic_and_autograd():
    inp = flp_inputs.make_embedding_inputs(5000, 128, 3000, BF16, 50, ids="zipf",
                                           invalid=(-1, 3000))
    m = flp()
    a = run(inp)[1]
    b = run(inp)[1]
    w = inp["weight"].cuda().requires_grad_(True)
    ids = inp["ids"].cuda()
    out = m.embedding(w, ids)
    (out.float() * inp["grad"].cuda().float()).sum().backward()
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert torch.equal(w.grad, a)


def test_embedding_full_shape():
    """The model row's shape: N = 16384 tokens, D = 2688, V = 131072 (bf16).  The lookup is
    exact; d_weight rows of every id that occurs (and a sample of absent ids) against the
    oracle; d_weight's column sums equal the sum of the valid gradient rows."""
    N, D, V = 16384, 2688, 131072
    inp = flp_inputs.make_embedding_inputs(N, D, V, BF16, 51, ids="zipf", invalid=(-1, V),
                                           device="cuda:0")
    inp["ids"] = inp["ids"].cuda()
    m = flp()
    out = m.embedding_forward(inp["weight"], inp["ids"])
    dw = m.embedding_backward(inp["grad"], inp["ids"], V)
    torch.cuda.synchronize()
    ids = inp["ids"]
    ok = (ids >= 0) & (ids < V)
    assert torch.equal(out[ok], inp["weight"][ids[ok]])
    assert not out[~ok].any()
    present = torch.unique(ids[ok])
    say(f"{int(present.numel())} distinct ids among {N} tokens")
    g_cpu, ids_cpu = inp["grad"].cpu(), ids.cpu()
    ref = oracle.embedding_backward(g_cpu, ids_cpu, V)
    rows = present.cpu()
    check_close("d_weight (present ids)", dw[present].float(), ref[rows.numpy()],
                **REDUCTION_CELL)
    absent = torch.ones(V, dtype=torch.bool, device="cuda:0")
    absent[present] = False
    assert not dw[absent].any()
