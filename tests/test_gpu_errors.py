"""Fail-closed behaviour on the GPU, through the C ABI with real device buffers:
every bad call returns its status and leaves the outputs untouched."""
import pytest
import torch

from gpu_common import flp

pytestmark = pytest.mark.gpu


def _bufs(N=64, D=128, V=500, dtype=torch.bfloat16):
    d = "cuda:0"
    return dict(h=torch.randn(N, D, device=d).to(dtype), w=torch.randn(V, D, device=d).to(dtype),
                t=torch.randint(0, V, (N,), device=d), lp=torch.full((N,), 7.0, device=d),
                ls=torch.full((N,), 7.0, device=d), N=N, D=D, V=V)


def _fwd(b, **kw):
    m = flp()
    a = dict(N=b["N"], D=b["D"], V=b["V"], x=m.FLP_BF16, h=b["h"].data_ptr(), w=b["w"].data_ptr(),
             t=b["t"].data_ptr(), lp=b["lp"].data_ptr(), ls=b["ls"].data_ptr())
    a.update(kw)
    wsb = m.flp_forward_workspace_bytes(a["N"], a["D"], a["V"]) if a["N"] >= 0 else 0
    ws = torch.empty(max(wsb, 256) + 4096, dtype=torch.uint8, device="cuda:0")
    wsb = kw.get("wsb", wsb)
    st = m.flp_forward(a["N"], a["D"], a["V"], a["x"], a["h"], a["w"], 0, a["t"], m.FLP_I64, 0,
                       a["lp"], a["ls"], kw.get("ws", ws.data_ptr()), wsb,
                       torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return m._abi.STATUS_NAMES[st]


def test_ok_then_errors_leave_outputs_untouched():
    b = _bufs()
    assert _fwd(b) == "FLP_OK"
    assert torch.all(b["lp"] <= 0) and torch.isfinite(b["ls"]).all()
    b = _bufs()
    cases = [
        (dict(h=b["h"].data_ptr() + 2), "FLP_MISALIGNED"),
        (dict(D=96), "FLP_OK"),   # smaller D over the same buffers is legal
        (dict(D=100), "FLP_UNSUPPORTED_SHAPE"),
        (dict(x=7), "FLP_UNSUPPORTED_DTYPE"),
        (dict(wsb=64), "FLP_WORKSPACE_TOO_SMALL"),
        (dict(lp=b["h"].data_ptr()), "FLP_INVALID_ARGUMENT"),
        (dict(ws=b["w"].data_ptr()), "FLP_INVALID_ARGUMENT"),
    ]
    for kw, expect in cases:
        if expect != "FLP_OK":
            before = b["lp"].clone()
            assert _fwd(b, **kw) == expect, kw
            assert torch.equal(b["lp"], before), kw


def test_empty_batch_is_a_noop():
    m = flp()
    st = m.flp_forward(0, 128, 500, m.FLP_BF16, 0, 0, 0, 0, m.FLP_I64, 0, 0, 0, 0, 0, 0)
    assert st == m.FLP_OK
    h = torch.empty(0, 128, dtype=torch.bfloat16, device="cuda:0")
    w = torch.randn(500, 128, device="cuda:0").to(torch.bfloat16)
    t = torch.empty(0, dtype=torch.int64, device="cuda:0")
    lp, ls = m.forward(h, w, t)
    assert lp.shape == (0,) and ls.shape == (0,)


def test_empty_batch_zeroes_the_sums():
    """N = 0: the backward calls write d_weight and d_bias as zeros (sums over no rows)."""
    m = flp()
    d = "cuda:0"
    D, V = 128, 500
    s = torch.cuda.current_stream().cuda_stream
    w = torch.randn(V, D, device=d).to(torch.bfloat16)
    for dwt, code in ((torch.bfloat16, m.FLP_BF16), (torch.float32, m.FLP_F32)):
        dw = torch.full((V, D), 7.0, device=d, dtype=dwt)
        db = torch.full((V,), 7.0, device=d)
        st = m.flp_backward(0, D, V, m.FLP_BF16, 0, 0, 0, w.data_ptr(), 0, 0, m.FLP_I64, 0, 0,
                            dw.data_ptr(), code, db.data_ptr(), 0, 0, s)
        torch.cuda.synchronize()
        assert st == m.FLP_OK and not dw.any() and not db.any()
        dw.fill_(7.0)
        db.fill_(7.0)
        st = m.flp_backward_indexed(0, D, V, m.FLP_BF16, 0, 0, 0, w.data_ptr(), 0, 0, m.FLP_I64,
                                    0, 0, m.FLP_I64, 0, 0, dw.data_ptr(), code, db.data_ptr(), 0,
                                    0, s)
        torch.cuda.synchronize()
        assert st == m.FLP_OK and not dw.any() and not db.any()
        dw.fill_(7.0)
        st = m.flp_embedding_backward(0, D, V, m.FLP_BF16, 0, 0, m.FLP_I64, dw.data_ptr(), code,
                                      0, 0, s)
        torch.cuda.synchronize()
        assert st == m.FLP_OK and not dw.any()
    # the same through the torch layer
    h = torch.empty(0, D, dtype=torch.bfloat16, device=d)
    t = torch.empty(0, dtype=torch.int64, device=d)
    z = torch.empty(0, device=d)
    b = torch.randn(V, device=d)
    dh, dw, db = m.backward(z, z, h, w, t, b)
    torch.cuda.synchronize()
    assert dh.shape == (0, D) and not dw.any() and not db.any()
    assert not m.embedding_backward(h, t, V).any()


def test_python_layer_rejects_bad_tensors():
    m = flp()
    b = _bufs()
    with pytest.raises(TypeError):
        m.forward(b["h"], b["w"].float(), b["t"])
    with pytest.raises(ValueError):
        m.forward(b["h"].t(), b["w"], b["t"])
    with pytest.raises(m.FlpError):
        m.forward(b["h"][:, :100].contiguous(), b["w"][:, :100].contiguous(), b["t"])
