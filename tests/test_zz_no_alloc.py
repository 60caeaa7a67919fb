"""The allocation-free forward (flp_forward_noalloc) through the C ABI.

Its outputs must equal flp_forward's bit for bit (same kernels, only the
workspace differs) on consecutive calls whose sizes shrink: the fixed per-device
array keeps the previous call's contents, which the next call must not depend
on.  The largest batch of the rollout shape fits the array; a larger one is
rejected before anything is enqueued."""
import pytest
import torch

import flp_inputs
from gpu_common import flp, inputs, say, to_gpu

pytestmark = pytest.mark.gpu


def _ptr(t):
    return 0 if t is None else int(t.data_ptr())


def _xdt(m, dtype):
    return {torch.bfloat16: m.FLP_BF16, torch.float16: m.FLP_F16, torch.float32: m.FLP_F32}[dtype]


def _both(m, g, with_lse=True):
    """flp_forward (caller workspace) and flp_forward_noalloc on the same inputs."""
    D = g["hidden"].shape[-1]
    N = g["hidden"].numel() // D
    V = g["weight"].shape[0]
    x = _xdt(m, g["hidden"].dtype)
    t64 = m.FLP_I64 if g["targets"].dtype == torch.int64 else m.FLP_I32
    s = torch.cuda.current_stream().cuda_stream
    dev = g["hidden"].device
    ref_lp = torch.full((N,), float("nan"), device=dev)
    ref_ls = torch.full((N,), float("nan"), device=dev) if with_lse else None
    ws = torch.empty(m.flp_forward_workspace_bytes(N, D, V), dtype=torch.uint8, device=dev)
    st = m.flp_forward(N, D, V, x, _ptr(g["hidden"]), _ptr(g["weight"]), _ptr(g["bias"]),
                       _ptr(g["targets"]), t64, _ptr(g["temperature"]), _ptr(ref_lp),
                       _ptr(ref_ls), _ptr(ws), ws.numel(), s)
    assert st == m.FLP_OK, m.flp_status_string(st)
    lp = torch.full((N,), float("nan"), device=dev)
    ls = torch.full((N,), float("nan"), device=dev) if with_lse else None
    st = m.flp_forward_noalloc(N, D, V, x, _ptr(g["hidden"]), _ptr(g["weight"]), _ptr(g["bias"]),
                               _ptr(g["targets"]), t64, _ptr(g["temperature"]), _ptr(lp), _ptr(ls),
                               s)
    assert st == m.FLP_OK, m.flp_status_string(st)
    torch.cuda.synchronize()
    return (ref_lp, ref_ls), (lp, ls)


def test_noalloc_equals_forward_on_shrinking_calls():
    m = flp()
    cases = []
    # 1: the full rollout batch (8192 rows, D = 2688, V = 131072, per-row temperature): the
    #    largest batch of the shape: 33,587,200 workspace bytes of the 34,603,008-byte array
    cases.append(("rollout_n8192 (8192 rows)", to_gpu(inputs("rollout_n8192")), True))
    # 2: the decode batch (32 rows of the same shape), rollout entry (no lse)
    cases.append(("decode_n32 (32 rows, no lse)", to_gpu(inputs("decode_n32")), False))
    # 3: a small ragged fp16 batch with bias, temperature, ignored rows and int32 targets
    w = flp_inputs.Workload("noalloc_small", 41, 77, 320, 3001, torch.float16, w_std=0.07,
                            bias_std=0.1, n_ignored=5, ignore_values=(-1, 3001),
                            temperature=(0.5, 1.5), grad="normal", leading=(77,))
    inp = flp_inputs.make_inputs(w)
    inp["targets"] = inp["targets"].to(torch.int32)
    cases.append(("fp16 77 x 320 x 3001 with bias", to_gpu(inp), True))
    for name, g, with_lse in cases:
        say(f"noalloc case: {name}")
        (rlp, rls), (lp, ls) = _both(m, g, with_lse)
        assert torch.isfinite(rlp).all()
        assert torch.equal(lp, rlp), name
        if with_lse:
            assert torch.equal(ls, rls), name
        del g


def test_noalloc_rejects_batches_beyond_the_array():
    """8440 rows at V = 131072 need more workspace than the fixed array: the call
    returns FLP_WORKSPACE_TOO_SMALL and leaves the outputs untouched."""
    m = flp()
    N, D, V = 8440, 64, 131072
    dev = "cuda:0"
    h = torch.zeros(N, D, dtype=torch.bfloat16, device=dev)
    w = torch.zeros(V, D, dtype=torch.bfloat16, device=dev)
    t = torch.zeros(N, dtype=torch.int64, device=dev)
    lp = torch.full((N,), 7.0, device=dev)
    st = m.flp_forward_noalloc(N, D, V, m.FLP_BF16, _ptr(h), _ptr(w), 0, _ptr(t), m.FLP_I64, 0,
                               _ptr(lp), 0, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert m._abi.STATUS_NAMES[st] == "FLP_WORKSPACE_TOO_SMALL"
    assert torch.all(lp == 7.0)
    # the empty batch is a no-op
    assert m.flp_forward_noalloc(0, D, V, m.FLP_BF16, 0, _ptr(w), 0, 0, m.FLP_I64, 0, 0, 0, 0) == \
        m.FLP_OK
