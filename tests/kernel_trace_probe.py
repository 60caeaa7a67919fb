"""Child program of test_gpu_kernels.py's kernel-trace test (not collected by pytest).

Prepares one small training-shaped batch on the GPU, then calls flp_forward and
flp_backward through the C ABI on preallocated buffers, so that between the
library's first and last kernel no other kernel is launched: a kernel trace of
this process then shows exactly the kernels the two calls run."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import torch  # noqa: E402

import flp_inputs  # noqa: E402
import lm_head_selected_bf16_amd as m  # noqa: E402


def main() -> None:
    m.load()
    inp = flp_inputs.make_inputs("train_n16384", n_rows=600)
    g = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    N, D = g["hidden"].shape
    V = g["weight"].shape[0]
    p = lambda t: 0 if t is None else int(t.data_ptr())  # noqa: E731
    logp = torch.empty(N, device="cuda")
    lse = torch.empty(N, device="cuda")
    dh = torch.empty_like(g["hidden"])
    dw = torch.empty_like(g["weight"])
    db = torch.empty(V, device="cuda")
    fws = torch.empty(m.flp_forward_workspace_bytes(N, D, V), dtype=torch.uint8, device="cuda")
    bwb = m.flp_backward_workspace_bytes(N, D, V, m.FLP_BF16, m.FLP_BF16, 0)
    bws = torch.empty(bwb, dtype=torch.uint8, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    torch.cuda.synchronize()
    st = m.flp_forward(N, D, V, m.FLP_BF16, p(g["hidden"]), p(g["weight"]), p(g["bias"]),
                       p(g["targets"]), m.FLP_I64, p(g["temperature"]), p(logp), p(lse), p(fws),
                       fws.numel(), s)
    assert st == m.FLP_OK, m.flp_status_string(st)
    st = m.flp_backward(N, D, V, m.FLP_BF16, p(g["grad_out"]), p(lse), p(g["hidden"]),
                        p(g["weight"]), p(g["bias"]), p(g["targets"]), m.FLP_I64,
                        p(g["temperature"]), p(dh), p(dw), m.FLP_BF16, p(db), p(bws), bws.numel(), s)
    assert st == m.FLP_OK, m.flp_status_string(st)
    torch.cuda.synchronize()
    print(f"kernel trace probe done: N={N} D={D} V={V}, {m.flp_build_info()[:60]}", flush=True)


if __name__ == "__main__":
    main()
