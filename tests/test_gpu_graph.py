"""The operator inside a captured HIP graph: flp_forward + flp_backward, and
flp_forward_noalloc, recorded once and replayed with new inputs.

The library enqueues only kernels on the caller's stream (no memset, no host
synchronisation, no allocation once a call's buffers are given), so a capture
replays the same work.  Every replay, with the program's own eager work and
synchronisations between replays, must equal the eager calls on the same inputs
bit for bit (PR #555, "Acceptance checks": repeat runs are bitwise identical)."""
import numpy as np
import pytest
import torch

import flp_inputs
from gpu_common import flp, say, to_gpu

pytestmark = pytest.mark.gpu
BF16 = torch.bfloat16


def _case():
    w = flp_inputs.Workload("graph_small", 57, 300, 512, 4133, BF16, w_std=1.3 / np.sqrt(512),
                            bias_std=0.1, n_ignored=5, ignore_values=(-1, 4133, -7, 4136),
                            temperature=(0.5, 1.5), grad="normal", leading=(300,))
    return to_gpu(flp_inputs.make_inputs(w))


def _fwd_bwd(m, g):
    lp, ls = m.forward(g["hidden"], g["weight"], g["targets"], g["bias"], g["temperature"])
    dh, dw, db = m.backward(g["grad_out"], ls, g["hidden"], g["weight"], g["targets"], g["bias"],
                            g["temperature"], need_bias=True)
    return lp, ls, dh, dw, db


def _new_hidden(g, seed):
    gen = torch.Generator(device="cpu").manual_seed(seed)
    h = torch.randn(g["hidden"].shape, generator=gen) * float(g["hidden"].float().std())
    return h.to(g["hidden"].dtype).to(g["hidden"].device)


def _capture(fn):
    """Warm up on a side stream (kernel attributes are set on first use), then capture."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = fn()
    torch.cuda.synchronize()
    return graph, out


def test_forward_backward_graph_replays():
    m = flp()
    m.flp_profile_enable(False)
    g = _case()
    graph, out = _capture(lambda: _fwd_bwd(m, g))
    for rep in range(4):
        if rep >= 2:  # new hidden rows and upstream gradients in the captured input buffers
            g["hidden"].copy_(_new_hidden(g, 100 + rep))
            g["grad_out"].copy_(torch.randn(g["grad_out"].shape,
                                            generator=torch.Generator().manual_seed(rep)).cuda())
        graph.replay()
        torch.cuda.synchronize()
        ref = _fwd_bwd(m, g)  # eager, on the same inputs
        torch.cuda.synchronize()
        for name, a, b in zip(("logp", "lse", "d_hidden", "d_weight", "d_bias"), out, ref):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager call"
        say(f"replay {rep}: forward + backward equal the eager calls bit for bit")


def test_noalloc_forward_graph_replays():
    m = flp()
    m.flp_profile_enable(False)
    g = _case()
    D = g["hidden"].shape[-1]
    N, V = g["hidden"].numel() // D, g["weight"].shape[0]
    lp = torch.empty(N, device="cuda")
    ls = torch.empty(N, device="cuda")

    def call():
        st = m.flp_forward_noalloc(N, D, V, m.FLP_BF16, g["hidden"].data_ptr(),
                                   g["weight"].data_ptr(), g["bias"].data_ptr(),
                                   g["targets"].data_ptr(), m.FLP_I64,
                                   g["temperature"].data_ptr(), lp.data_ptr(), ls.data_ptr(),
                                   torch.cuda.current_stream().cuda_stream)
        assert st == m.FLP_OK, m.flp_status_string(st)
        return lp, ls

    graph, _ = _capture(call)
    for rep in range(4):
        if rep >= 2:
            g["hidden"].copy_(_new_hidden(g, 200 + rep))
        lp.fill_(float("nan"))
        ls.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        rl, rs = m.forward(g["hidden"], g["weight"], g["targets"], g["bias"], g["temperature"])
        torch.cuda.synchronize()
        assert torch.equal(lp, rl) and torch.equal(ls, rs), f"replay {rep} differs"
        say(f"replay {rep}: the allocation-free forward equals flp_forward bit for bit")
