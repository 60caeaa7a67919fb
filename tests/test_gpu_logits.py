"""The operator on materialised logits (flp_logits_forward / flp_logits_backward)
against the FP64 oracle (oracle.logits_forward / logits_backward), bitwise row
independence, and the autograd wrapper.  PR #234 "Summary" / "Implementation
details" and PR #547 "What" fix the definitions; the docs page's intro contrasts
this operator with the linear one."""
import numpy as np
import pytest
import torch

import flp_inputs
import oracle
from gpu_common import FP32_CELL, LOGP_CELL, check_close, flp, say

pytestmark = pytest.mark.gpu


def run(inp, device="cuda:0"):
    m = flp()
    z = inp["logits"].to(device)
    t = inp["targets"].to(device)
    g = inp["grad_out"].to(device)
    logp, lse = m.logits_forward(z, t)
    d = m.logits_backward(g, lse, z, t)
    return logp, lse, d


CASES = [
    # (dtype, N, V, n_ignored, target dtype)
    (torch.bfloat16, 300, 4136, 7, torch.int64),
    (torch.float16, 77, 1000, 3, torch.int32),
    (torch.float32, 64, 4100, 4, torch.int64),
    (torch.bfloat16, 1, 8, 0, torch.int64),
]


@pytest.mark.parametrize("k", range(len(CASES)))
def test_logits_op_parity(k):
    dtype, N, V, nign, tdt = CASES[k]
    say(f"logits case {k}: {dtype} N={N} V={V}")
    inp = flp_inputs.make_logits_inputs(f"logits{k}", N, V, dtype, 50 + k, n_ignored=nign,
                                        ignore_values=(-1, V, -5, V + 9), logit_std=2.0)
    inp["targets"] = inp["targets"].to(tdt)
    logp, lse, d = run(inp)
    rl, rs = oracle.logits_forward(inp["logits"], inp["targets"])
    rd = oracle.logits_backward(inp["logits"], inp["targets"], inp["grad_out"])
    cell = FP32_CELL if dtype == torch.float32 else LOGP_CELL
    check_close("logp", logp, rl, **cell)
    check_close("lse", lse, rs, **cell)
    check_close("d_logits", d.float(), rd, **cell)
    t = inp["targets"].long().numpy()
    ign = (t < 0) | (t >= V)
    assert np.all(logp.cpu().numpy()[ign] == 0.0)
    assert np.all(d.float().cpu().numpy()[ign] == 0.0)


def test_logits_op_row_subsets_bitwise():
    inp = flp_inputs.make_logits_inputs("logits_inv", 1000, 2048, torch.bfloat16, 60,
                                        n_ignored=5, ignore_values=(-1, 2048))
    logp, lse, d = run(inp)
    for n in (1, 7, 257):
        rows = flp_inputs.random_rows(1000, n, seed=600 + n)
        sub = {k: (v[rows].contiguous() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
        lp, ls, dd = run(sub)
        idx = rows.to(logp.device)
        assert torch.equal(lp, logp[idx]) and torch.equal(ls, lse[idx]) and torch.equal(dd, d[idx])


def test_logits_op_autograd():
    m = flp()
    inp = flp_inputs.make_logits_inputs("logits_ag", 40, 520, torch.bfloat16, 61, n_ignored=2)
    z = inp["logits"].cuda().requires_grad_(True)
    t = inp["targets"].cuda()
    g = inp["grad_out"].cuda()
    logp = m.logits_logp(z, t)
    (logp * g).sum().backward()
    _, lse = m.logits_forward(z.detach(), t)
    assert torch.equal(z.grad, m.logits_backward(g, lse, z.detach(), t))


def test_logits_op_large_sampled():
    """N=8192 rows of V=131072 bf16 logits (2.1 GB): every row's logp/lse and 16 sampled rows
    of d_logits against the oracle."""
    N, V = 8192, 131072
    inp = flp_inputs.make_logits_inputs("logits_n8192", N, V, torch.bfloat16, 62, n_ignored=64,
                                        ignore_values=(-1, V), device="cuda:0")
    logp, lse, d = run(inp)
    rows = flp_inputs.random_rows(N, 16, seed=620).numpy()
    z_rows = inp["logits"][torch.as_tensor(rows, device="cuda:0")].cpu()
    t_rows = inp["targets"][rows]
    rl, rs = oracle.logits_forward(z_rows, t_rows)
    rd = oracle.logits_backward(z_rows, t_rows, inp["grad_out"][rows])
    idx = torch.as_tensor(rows, device="cuda:0")
    check_close("logp (sampled)", logp[idx], rl, **LOGP_CELL)
    check_close("lse (sampled)", lse[idx], rs, **LOGP_CELL)
    check_close("d_logits (sampled)", d[idx].float(), rd, **LOGP_CELL)
    # every row: the softmax of a row sums to one, i.e. sum_v exp(z - lse) = 1 (fp64 on the GPU)
    s = torch.exp(inp["logits"].double() - lse.double()[:, None]).sum(dim=1)
    assert float((s - 1).abs().max()) < 1e-4
