"""Shared helpers of the GPU tests: seeded inputs on the device, the HIP path
through the C ABI, oracle comparisons with the stated tolerances."""
from __future__ import annotations

import functools
import sys

import numpy as np
import torch

import flp_inputs
import oracle

# Tolerance cells (PR #555, "Tolerance" and summary bullets): the log-prob cell
# for logp, lse and d_hidden; the reduction cell for reductions over tokens
# (d_weight, d_bias).  fp32 inputs: 1e-4 absolute on everything.
LOGP_CELL = dict(atol=0.05, rtol=0.0)
REDUCTION_CELL = dict(atol=0.1, rtol=0.02)
FP32_CELL = dict(atol=1e-4, rtol=0.0)


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def flp():
    import lm_head_selected_bf16_amd as m
    m.load()
    return m


def dev(x, device="cuda:0"):
    return None if x is None else x.to(device)


@functools.lru_cache(maxsize=2)
def workload_weight(name: str) -> torch.Tensor:
    return flp_inputs.draw_weight(flp_inputs.WORKLOADS[name])


def inputs(name: str, n_rows=None):
    """CPU inputs of a workload (W cached across calls)."""
    return flp_inputs.make_inputs(name, n_rows=n_rows, weight=workload_weight(name))


def to_gpu(inp):
    return {k: (dev(v) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def gpu_forward(g, return_lse=True):
    m = flp()
    return m.forward(g["hidden"], g["weight"], g["targets"], g["bias"], g["temperature"],
                     return_lse=return_lse)


def gpu_backward(g, lse, grad_out=None, **kw):
    m = flp()
    go = g["grad_out"] if grad_out is None else grad_out
    return m.backward(go, lse, g["hidden"], g["weight"], g["targets"], g["bias"], g["temperature"], **kw)


def check_close(name, got, ref, atol, rtol):
    got = got.detach().to("cpu").double().numpy() if hasattr(got, "detach") else np.asarray(got)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    err = np.abs(got - ref)
    bound = atol + rtol * np.abs(ref)
    bad = err > bound
    worst = float(err.max()) if err.size else 0.0
    say(f"  {name}: max|err| = {worst:.3e} (atol {atol}, rtol {rtol}), "
        f"{int(bad.sum())} of {err.size} outside")
    assert not bad.any(), f"{name}: {int(bad.sum())} elements outside the tolerance, max err {worst}"
    return worst


def oracle_forward(inp, rows=None):
    return oracle.forward(inp["hidden"], inp["weight"], inp["targets"], inp["bias"],
                          inp["temperature"], rows=rows)


def oracle_backward(inp, grad_out=None, rows=None, need_weight=True, need_bias=True):
    go = inp["grad_out"] if grad_out is None else grad_out
    return oracle.backward(inp["hidden"], inp["weight"], inp["targets"], go, inp["bias"],
                           inp["temperature"], rows=rows, need_weight=need_weight,
                           need_bias=need_bias)


_FLP_X = {torch.bfloat16: 0, torch.float32: 1, torch.float16: 4}


def workspace_for_chunk(N, D, V, x_dtype, dw_dtype, rows, need_hidden=True, need_weight=True,
                        need_bias=True):
    """The smallest backward workspace with which flp_backward processes `rows` rows per
    chunk for the requested outputs (found with the library's host-side planner,
    flp_backward_chunk_rows, which picks the largest chunk that fits)."""
    from lm_head_selected_bf16_amd import _abi
    x, dw = _FLP_X[x_dtype], _FLP_X[dw_dtype]

    def chunk(b):
        return _abi.flp_backward_chunk_rows(N, D, V, x, dw, b, need_hidden, need_weight, need_bias)

    lo, hi = 0, 1 << 40
    while lo < hi:  # smallest workspace whose chunk is at least `rows`
        mid = (lo + hi) // 2
        if chunk(mid) >= rows:
            hi = mid
        else:
            lo = mid + 1
    assert chunk(lo) == rows, (rows, chunk(lo))
    return lo
