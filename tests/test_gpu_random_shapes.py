"""Parity against the FP64 oracle over drawn shapes: N, D (a multiple of 32), V,
input dtype, bias, temperature and target dtype vary together, so ragged row,
vocabulary and K tiles meet in combinations the fixed cases do not list.  The
draws are derandomized: every run checks the same examples.  Operation and
tolerances as in test_gpu_parity.py (docs page "Fused Linear LogP", Reference
Semantics; PR #555 Tolerance)."""
import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import flp_inputs
from gpu_common import (FP32_CELL, LOGP_CELL, REDUCTION_CELL, check_close, gpu_backward,
                        gpu_forward, oracle_backward, oracle_forward, say, to_gpu)

pytestmark = pytest.mark.gpu

DTYPES = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


@settings(max_examples=16, deadline=None, derandomize=True, database=None)
@given(N=st.integers(1, 600), dk=st.integers(1, 16), V=st.integers(1, 2100),
       dt=st.sampled_from(sorted(DTYPES)), bias=st.booleans(), temp=st.booleans(),
       t32=st.booleans(), seed=st.integers(0, 1000))
def test_random_shapes_parity(N, dk, V, dt, bias, temp, t32, seed):
    D = 32 * dk
    dtype = DTYPES[dt]
    say(f"random shape: N={N} D={D} V={V} {dt} bias={bias} T={temp} int32={t32} seed={seed}")
    w = flp_inputs.Workload(f"rand{seed}", 500 + seed, N, D, V, dtype,
                            w_std=1.3 / np.sqrt(D), bias_std=0.1 if bias else None,
                            n_ignored=min(3, N // 4), ignore_values=(-1, V, -9, V + 5),
                            temperature=(0.5, 1.5) if temp else None, grad="normal",
                            leading=(N,))
    inp = flp_inputs.make_inputs(w)
    if t32:
        inp["targets"] = inp["targets"].to(torch.int32)
    g = to_gpu(inp)
    lp, ls = gpu_forward(g)
    dh, dW, db = gpu_backward(g, ls, need_bias=bias)
    rl, rs = oracle_forward(inp)
    rdh, rdw, rdb = oracle_backward(inp, need_bias=bias)
    cell = FP32_CELL if dtype == torch.float32 else LOGP_CELL
    red = FP32_CELL if dtype == torch.float32 else REDUCTION_CELL
    check_close("logp", lp, rl, **cell)
    check_close("lse", ls, rs, **cell)
    check_close("d_hidden", dh.float(), rdh, **cell)
    check_close("d_weight", dW.float(), rdw, **red)
    if bias:
        check_close("d_bias", db, rdb, **red)


@settings(max_examples=12, deadline=None, derandomize=True, database=None)
@given(N=st.integers(1, 400), v8=st.integers(1, 400), dt=st.sampled_from(sorted(DTYPES)),
       indexed=st.booleans(), seed=st.integers(0, 1000))
def test_random_shapes_logits_op(N, v8, dt, indexed, seed):
    """The operator on given logits (V a multiple of 8: whole 16-byte chunks for every
    dtype), dense or with a drawn id list."""
    import oracle
    from gpu_common import flp

    V = 8 * v8
    dtype = DTYPES[dt]
    say(f"random logits: N={N} V={V} {dt} indexed={indexed} seed={seed}")
    inp = flp_inputs.make_logits_inputs(f"rl{seed}", N, V, dtype, 700 + seed,
                                        n_ignored=min(2, N // 4), ignore_values=(-1, V),
                                        logit_std=2.0)
    m = flp()
    z, t, go = inp["logits"].cuda(), inp["targets"].cuda(), inp["grad_out"].cuda()
    cell = FP32_CELL if dtype == torch.float32 else LOGP_CELL
    if indexed:
        ids = flp_inputs.row_ids(N, max(N // 2, 1), seed=seed, n_dup=N // 8, invalid=(N,))
        lp, ls = m.logits_forward_indexed(z, t, ids.cuda())
        d = m.logits_backward_indexed(go, ls, z, t, ids.cuda())
        rl, rs = oracle.logits_forward_indexed(inp["logits"], inp["targets"], ids)
        rd = oracle.logits_backward_indexed(inp["logits"], inp["targets"], inp["grad_out"], ids)
    else:
        lp, ls = m.logits_forward(z, t)
        d = m.logits_backward(go, ls, z, t)
        rl, rs = oracle.logits_forward(inp["logits"], inp["targets"])
        rd = oracle.logits_backward(inp["logits"], inp["targets"], inp["grad_out"])
    check_close("logp", lp, rl, **cell)
    check_close("lse", ls, rs, **cell)
    check_close("d_logits", d.float(), rd, **cell)


@settings(max_examples=12, deadline=None, derandomize=True, database=None)
@given(N=st.integers(1, 3000), dk=st.integers(1, 12), V=st.integers(1, 5000),
       dt=st.sampled_from(sorted(DTYPES)), draw=st.sampled_from(["zipf", "uniform", "same"]),
       f32_dw=st.booleans(), seed=st.integers(0, 1000))
def test_random_shapes_embedding(N, dk, V, dt, draw, f32_dw, seed):
    """The embedding lookup (exact) and its grad_weight against the oracle."""
    import oracle
    from gpu_common import flp

    D = 8 * dk
    dtype = DTYPES[dt]
    dwt = torch.float32 if (f32_dw or dtype == torch.float32) else None
    say(f"random embedding: N={N} D={D} V={V} {dt} ids {draw} dW fp32={dwt is not None}")
    inp = flp_inputs.make_embedding_inputs(N, D, V, dtype, 800 + seed, ids=draw, invalid=(-1, V))
    m = flp()
    w, ids, g = inp["weight"].cuda(), inp["ids"].cuda(), inp["grad"].cuda()
    out = m.embedding_forward(w, ids)
    dw = m.embedding_backward(g, ids, V, dw_dtype=dwt)
    torch.cuda.synchronize()
    assert torch.equal(out.double().cpu(), torch.from_numpy(oracle.embedding_forward(inp["weight"], inp["ids"])))
    cell = FP32_CELL if dwt is not None else REDUCTION_CELL
    check_close("d_weight", dw.float(), oracle.embedding_backward(inp["grad"], inp["ids"], V), **cell)
