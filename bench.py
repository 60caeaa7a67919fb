#!/usr/bin/env python3
"""Throughput of the fused linear selected-token log-prob on one MI355X.

One step = flp_forward + flp_backward (logp, lse, d_hidden, d_weight, d_bias)
over the training workload N = 16384 tokens (B = 4, S = 4096), D = 2688,
V = 131072, bf16 hidden/W, fp32 bias, grad_out ~ N(0, 1); d_weight in bf16
from fp32 accumulation.  Inputs are synthetic (seeded; see flp_inputs.py) and
resident in HBM before the timed region; outputs and workspaces are
preallocated.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Roofline: per-kernel durations come from HIP events the library records around
each of its launches during the timed steps (flp_profile_*); the dominant
kernel's algorithmic flops per launch (2 N D V for a full-batch launch of any
of the four contractions) over its mean duration, against the bf16 dense MFMA
peak.  cpu_baseline: the CPU FP64 oracle, as it stands, on a bounded sample of
rows of the same workload, scaled to tokens/s.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
# The pages' own number for this exact workload on other hardware (H100 PCIe,
# strict deterministic path, cuBLASLt no-split-K): 351.2 ms per fwd+bwd at 16384 tokens.
PAGES_STRICT_TOK_S = 16384 / 0.3512


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_sha() -> str:
    p = os.path.join(ROOT, "lm_head_selected_bf16_amd", "csrc", "flp_kernels.hip")
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def load_traffic(workload: str, kernel: str):
    """HBM bytes per launch from the committed rocprofv3 PMC summary, if it was
    taken on the current kernel source (else None)."""
    p = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
    except Exception:  # noqa: BLE001
        return None
    if d.get("kernel_source_sha") != kernel_source_sha():
        return None
    k = d.get("kernels", {}).get(kernel)
    if not k:
        return None
    return k.get("hbm_bytes_per_launch")


class Problem:
    """Device buffers of one workload and raw C-ABI calls over them."""

    def __init__(self, name: str, backward: bool):
        import torch

        import flp_inputs
        import lm_head_selected_bf16_amd as m

        self.m = m
        self.torch = torch
        inp = flp_inputs.make_inputs(name)
        self.cpu = inp
        w = inp["workload"]
        self.w = w
        self.N, self.D, self.V = w.N, w.D, w.V
        dev = "cuda:0"
        g = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
        self.g = g
        self.x = m.FLP_BF16 if w.dtype == torch.bfloat16 else m.FLP_F32
        self.logp = torch.empty(self.N, device=dev)
        self.lse = torch.empty(self.N, device=dev)
        fb = m.flp_forward_workspace_bytes(self.N, self.D, self.V)
        self.fws = torch.empty(fb, dtype=torch.uint8, device=dev)
        self.backward = backward
        if backward:
            self.dh = torch.empty_like(g["hidden"])
            self.dw = torch.empty_like(g["weight"])
            self.db = torch.empty(self.V, device=dev)
            bb = m.default_backward_workspace_bytes(self.N, self.D, self.V, w.dtype)
            self.bws = torch.empty(bb, dtype=torch.uint8, device=dev)
        self.stream = torch.cuda.current_stream().cuda_stream

    def p(self, t):
        return 0 if t is None else int(t.data_ptr())

    def forward(self):
        g, m = self.g, self.m
        st = m.flp_forward(self.N, self.D, self.V, self.x, self.p(g["hidden"]), self.p(g["weight"]),
                           self.p(g["bias"]), self.p(g["targets"]), m.FLP_I64,
                           self.p(g["temperature"]), self.p(self.logp), self.p(self.lse),
                           self.p(self.fws), self.fws.numel(), self.stream)
        if st != m.FLP_OK:
            raise m.FlpError("flp_forward", st)

    def step(self):
        self.forward()
        if not self.backward:
            return
        g, m = self.g, self.m
        st = m.flp_backward(self.N, self.D, self.V, self.x, self.p(g["grad_out"]), self.p(self.lse),
                            self.p(g["hidden"]), self.p(g["weight"]), self.p(g["bias"]),
                            self.p(g["targets"]), m.FLP_I64, self.p(g["temperature"]),
                            self.p(self.dh), self.p(self.dw), self.x, self.p(self.db),
                            self.p(self.bws), self.bws.numel(), self.stream)
        if st != m.FLP_OK:
            raise m.FlpError("flp_backward", st)

    def time_steps(self, steps: int, warmup: int, profile: bool = True):
        """Time `steps` steps after `warmup` untimed ones.  With profile, the library's
        per-kernel HIP events are recorded inside the timed region (two event records per
        kernel launch); without, the region holds only the library's own launches."""
        torch, m = self.torch, self.m
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        m.flp_profile_read()          # drop anything recorded before
        m.flp_profile_enable(profile)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev[0].record()
        for k in range(steps):
            self.step()
            ev[k + 1].record()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        m.flp_profile_enable(False)
        prof = m.flp_profile_read()
        per = sorted(ev[k].elapsed_time(ev[k + 1]) for k in range(steps))
        self.step_ms_median, self.step_ms_min = per[len(per) // 2], per[0]
        return (t1 - t0) * 1e3 / steps, ev[0].elapsed_time(ev[steps]) / steps, prof


def contraction_flops(kind: str, N: int, D: int, V: int, launches_per_step: int) -> float:
    """Algorithmic flops per launch of a contraction kernel (rows split evenly
    over the launches of one step)."""
    if kind in ("forward", "dlogits", "d_hidden", "d_weight"):
        return 2.0 * N * D * V / launches_per_step
    return 0.0


def cpu_baseline(prob: Problem, target_s: float = 15.0):
    """The oracle on a bounded sample of rows: fwd + bwd (d_hidden, d_weight, d_bias)."""
    import numpy as np
    import threadpoolctl

    import flp_inputs
    import oracle

    inp = prob.cpu
    H = oracle.as_f64(inp["hidden"])
    W = oracle.as_f64(inp["weight"])          # up-cast once, outside the timed region
    b = oracle.as_f64(inp["bias"])
    T = oracle.as_f64(inp["temperature"])
    t = inp["targets"].numpy()
    g = inp["grad_out"].numpy()
    info = [i for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas"]
    threads = max([i.get("num_threads", 1) for i in info] or [1])

    def run(rows):
        t0 = time.perf_counter()
        oracle.forward(H, W, t, b, T, rows=rows)
        oracle.backward(H, W, t, g, b, T, rows=rows)
        return time.perf_counter() - t0

    # At least one whole 512-row chunk of the oracle: its d_weight update over
    # V x D is a fixed cost per chunk that a smaller sample would not amortise.
    probe = flp_inputs.random_rows(prob.N, 512, seed=5).numpy()
    dt = run(probe)
    n = int(min(2048, max(512, 512 * target_s / max(dt, 1e-3))))
    n -= n % 512
    if n > 512:
        log(f"cpu baseline: 512 rows took {dt:.2f}s -> timing {n} rows")
        rows = flp_inputs.random_rows(prob.N, n, seed=6).numpy()
        dt = run(rows)
    return {"value": n / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n} random rows of the {prob.w.name} workload (D={prob.D}, V={prob.V}), "
                      f"fwd + bwd (logp, lse, d_hidden, d_weight, d_bias) in float64 numpy, "
                      f"{dt:.1f} s; scaled to tokens/s (the oracle's work is linear in rows)",
            "host_cpus": os.cpu_count(), "affinity": len(os.sched_getaffinity(0))}


def cpu_oracle_configs():
    """The oracle's full runs on the small configurations: the fp32 tiny fwd+bwd and the
    decode forward (N = 32 rows of the full vocabulary)."""
    import threadpoolctl

    import flp_inputs
    import oracle

    info = [i for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas"]
    threads = max([i.get("num_threads", 1) for i in info] or [1])
    out = {"cores": int(threads), "kind": "oracle"}
    inp = flp_inputs.make_inputs("tiny_fp32")
    t0 = time.perf_counter()
    oracle.forward(inp["hidden"], inp["weight"], inp["targets"], inp["bias"], inp["temperature"])
    oracle.backward(inp["hidden"], inp["weight"], inp["targets"], inp["grad_out"], inp["bias"],
                    inp["temperature"])
    dt = time.perf_counter() - t0
    out["tiny_fp32_fwd_bwd"] = {"seconds": round(dt, 3), "tokens_per_s": round(64 / dt, 1)}
    inp = flp_inputs.make_inputs("decode_n32")
    t0 = time.perf_counter()
    oracle.forward(inp["hidden"], inp["weight"], inp["targets"], inp["bias"], inp["temperature"])
    dt = time.perf_counter() - t0
    out["decode_n32_fwd"] = {"seconds": round(dt, 3), "tokens_per_s": round(32 / dt, 1)}
    del inp
    # the rollout forward over all of its 8192 rows
    inp = flp_inputs.make_inputs("rollout_n8192")
    H, W = oracle.as_f64(inp["hidden"]), oracle.as_f64(inp["weight"])
    T = oracle.as_f64(inp["temperature"])
    t0 = time.perf_counter()
    oracle.forward(H, W, inp["targets"], inp["bias"], T)
    dt = time.perf_counter() - t0
    out["rollout_n8192_fwd"] = {"seconds": round(dt, 3), "tokens_per_s": round(8192 / dt, 1),
                                "rows": "all 8192"}
    del inp, H, W, T
    # the long sequence: a sample of 1024 of its 65600 rows, fwd + bwd (d_hidden, d_weight)
    inp = flp_inputs.make_inputs("longseq_n65600")
    H, W = oracle.as_f64(inp["hidden"]), oracle.as_f64(inp["weight"])
    t, g = inp["targets"].numpy(), inp["grad_out"].numpy()
    rows = flp_inputs.random_rows(65600, 1024, seed=8).numpy()
    t0 = time.perf_counter()
    oracle.forward(H, W, t, inp["bias"], inp["temperature"], rows=rows)
    oracle.backward(H, W, t, g, inp["bias"], inp["temperature"], rows=rows)
    dt = time.perf_counter() - t0
    out["longseq_n65600_fwd_bwd"] = {"seconds": round(dt, 3), "tokens_per_s": round(1024 / dt, 1),
                                     "rows": "a sample of 1024 random rows, scaled to tokens/s"}
    return out


def forward_only(name: str, steps: int, warmup: int, bound: str):
    import torch

    prob = Problem(name, backward=False)
    # the first call of this process on this workload, before any warm-up
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    prob.forward()
    e1.record()
    torch.cuda.synchronize()
    first_ms = e0.elapsed_time(e1)
    # the call as a caller sees it: no per-kernel events in the timed region
    ms, ems, _ = prob.time_steps(steps, warmup, profile=False)
    med, mn = prob.step_ms_median, prob.step_ms_min
    # the kernel breakdown from a separate pass with the library's per-kernel events on
    _, _, prof = prob.time_steps(steps, 1, profile=True)
    fwd_ms, fwd_n = prof["forward"]
    k_ms = fwd_ms / max(fwd_n, 1)
    out = {"workload": name, "N": prob.N, "ms_per_call": round(ms, 4),
           "ms_per_call_median": round(med, 4), "ms_per_call_min": round(mn, 4),
           "first_call_ms": round(first_ms, 4),
           "tokens_per_s": round(prob.N / (ms / 1e3), 1), "forward_kernel_ms": round(k_ms, 4),
           "merge_kernel_ms": round(prof["merge"][0] / max(prof["merge"][1], 1), 4),
           "timing": "ms_per_call and frac: whole calls (logit tiles + merge, launch gaps "
                     "included) with no per-kernel events; *_kernel_ms and *_kernel_frac: "
                     "per-kernel HIP events from a second pass"}
    if bound == "hbm":
        # algorithmic bytes: W + hidden read once, targets read, logp + lse written
        byts = prob.V * prob.D * 2 + prob.N * prob.D * 2 + prob.N * 8 + prob.N * 8
        gbs, kgbs = byts / (ms / 1e3) / 1e9, byts / (k_ms / 1e3) / 1e9
        out.update(bound="hbm", algorithmic_bytes=byts, achieved_GBs=round(gbs, 1),
                   peak_GBs=PEAK_HBM_GBS, frac=round(gbs / PEAK_HBM_GBS, 4),
                   frac_of_measured_peak=_meas_frac("hbm", gbs),
                   forward_kernel_GBs=round(kgbs, 1),
                   forward_kernel_frac=round(kgbs / PEAK_HBM_GBS, 4))
    else:
        fl = 2.0 * prob.N * prob.D * prob.V
        tf, ktf = fl / (ms / 1e3) / 1e12, fl / (k_ms / 1e3) / 1e12
        out.update(bound="mfma", algorithmic_flops=fl, achieved_TFLOPs=round(tf, 1),
                   peak_TFLOPs=PEAK_BF16_TFLOPS, frac=round(tf / PEAK_BF16_TFLOPS, 4),
                   frac_of_measured_peak=_meas_frac("mfma", tf),
                   forward_kernel_TFLOPs=round(ktf, 1),
                   forward_kernel_frac=round(ktf / PEAK_BF16_TFLOPS, 4))
    del prob
    return out


def shard_forward(name: str, shards: int, steps: int, warmup: int, bound: str):
    """flp_forward_partial over the first of `shards` equal vocabulary shards: the
    kernel at one rank's shape in a vocabulary tensor-parallel head."""
    import torch

    prob = Problem(name, backward=False)
    m, g = prob.m, prob.g
    V_local = prob.V // shards
    w = g["weight"][:V_local].contiguous()
    b = None if g["bias"] is None else g["bias"][:V_local].contiguous()
    part = torch.empty(m.flp_forward_partial_bytes(prob.N, V_local), dtype=torch.uint8,
                       device=w.device)
    zt = torch.empty(prob.N, dtype=torch.float32, device=w.device)

    def call():
        st = m.flp_forward_partial(prob.N, prob.D, V_local, 0, prob.V, prob.x, prob.p(g["hidden"]),
                                   prob.p(w), prob.p(b), prob.p(g["targets"]), m.FLP_I64,
                                   prob.p(g["temperature"]), prob.p(part), prob.p(zt), prob.stream)
        if st != m.FLP_OK:
            raise m.FlpError("flp_forward_partial", st)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    m.flp_profile_read()
    m.flp_profile_enable(True)
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    m.flp_profile_enable(False)
    tot, n = m.flp_profile_read()["forward"]
    k_ms = tot / max(n, 1)
    out = {"workload": name, "shards": shards, "V_local": V_local, "N": prob.N,
           "forward_kernel_ms": round(k_ms, 4)}
    if bound == "hbm":
        byts = V_local * prob.D * 2 + prob.N * prob.D * 2 + prob.N * 8 + prob.N * 4
        out.update(bound="hbm", algorithmic_bytes=byts,
                   achieved_GBs=round(byts / (k_ms / 1e3) / 1e9, 1), peak_GBs=PEAK_HBM_GBS,
                   frac=round(byts / (k_ms / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
                   frac_of_measured_peak=_meas_frac("hbm", byts / (k_ms / 1e3) / 1e9))
    else:
        fl = 2.0 * prob.N * prob.D * V_local
        out.update(bound="mfma", algorithmic_flops=fl,
                   achieved_TFLOPs=round(fl / (k_ms / 1e3) / 1e12, 1), peak_TFLOPs=PEAK_BF16_TFLOPS,
                   frac=round(fl / (k_ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                   frac_of_measured_peak=_meas_frac("mfma", fl / (k_ms / 1e3) / 1e12))
    del prob
    return out


def logits_op(N: int, V: int, steps: int, warmup: int):
    """The operator on materialised logits: flp_logits_forward and flp_logits_backward over
    N x V bf16 logits (HBM-bound: the forward reads them once, the backward reads them and
    writes d_logits)."""
    import torch

    import flp_inputs
    import lm_head_selected_bf16_amd as m

    inp = flp_inputs.make_logits_inputs("logits_bench", N, V, torch.bfloat16, 70, n_ignored=N // 64,
                                        ignore_values=(-1, V), device="cuda:0")
    z, t, g = inp["logits"], inp["targets"].cuda(), inp["grad_out"].cuda()
    logp = torch.empty(N, device="cuda:0")
    lse = torch.empty(N, device="cuda:0")
    d = torch.empty_like(z)
    stream = torch.cuda.current_stream().cuda_stream

    def call():
        st = m.flp_logits_forward(N, V, m.FLP_BF16, z.data_ptr(), t.data_ptr(), m.FLP_I64,
                                  logp.data_ptr(), lse.data_ptr(), stream)
        st2 = m.flp_logits_backward(N, V, m.FLP_BF16, g.data_ptr(), lse.data_ptr(), z.data_ptr(),
                                    t.data_ptr(), m.FLP_I64, d.data_ptr(), stream)
        if st != m.FLP_OK or st2 != m.FLP_OK:
            raise m.FlpError("flp_logits_forward/backward", st or st2)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    m.flp_profile_read()
    m.flp_profile_enable(True)
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    m.flp_profile_enable(False)
    prof = m.flp_profile_read()
    out = {"workload": f"logits_n{N}: given bf16 logits [{N}, {V}], fwd (logp, lse) + bwd (d_logits)"}
    for kind, byts in (("logits_forward", N * V * 2 + N * 16),
                       ("logits_backward", 2 * N * V * 2 + N * 16)):
        tot, n = prof[kind]
        k_ms = tot / max(n, 1)
        gbs = byts / (k_ms / 1e3) / 1e9
        out[kind] = {"kernel_ms": round(k_ms, 4), "bound": "hbm", "algorithmic_bytes": byts,
                     "achieved_GBs": round(gbs, 1), "peak_GBs": PEAK_HBM_GBS,
                     "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "frac_of_measured_peak": _meas_frac("hbm", gbs)}
    del z, d
    return out


def indexed_step(name: str, n_sel: int, steps: int, warmup: int):
    """flp_forward_indexed + flp_backward_indexed selecting n_sel of the workload's rows (a
    shuffled id list with repeats and out-of-range ids): the cost should follow the selected
    rows, plus the row selection, gather and scatter kernels."""
    import torch

    import flp_inputs

    prob = Problem(name, backward=False)
    m, g, N, D, V = prob.m, prob.g, prob.N, prob.D, prob.V
    ids = flp_inputs.row_ids(N, n_sel, seed=9, n_dup=n_sel // 16, invalid=(-1, N)).cuda()
    n_ids = int(ids.numel())
    fws = torch.empty(m.flp_forward_indexed_workspace_bytes(N, D, V, prob.x, n_ids),
                      dtype=torch.uint8, device="cuda:0")
    bws = torch.empty(m.flp_backward_indexed_workspace_bytes(N, D, V, prob.x, prob.x, n_ids,
                                                             min(n_ids, N)),
                      dtype=torch.uint8, device="cuda:0")
    dh = torch.empty_like(g["hidden"])
    dw = torch.empty_like(g["weight"])
    db = torch.empty(V, device="cuda:0")
    p = prob.p

    def call():
        st = m.flp_forward_indexed(N, D, V, prob.x, p(g["hidden"]), p(g["weight"]), p(g["bias"]),
                                   p(g["targets"]), m.FLP_I64, p(g["temperature"]), p(ids),
                                   m.FLP_I64, n_ids, p(prob.logp), p(prob.lse), p(fws),
                                   fws.numel(), prob.stream)
        st2 = m.flp_backward_indexed(N, D, V, prob.x, p(g["grad_out"]), p(prob.lse),
                                     p(g["hidden"]), p(g["weight"]), p(g["bias"]),
                                     p(g["targets"]), m.FLP_I64, p(g["temperature"]), p(ids),
                                     m.FLP_I64, n_ids, p(dh), p(dw), prob.x,
                                     p(db if g["bias"] is not None else None), p(bws),
                                     bws.numel(), prob.stream)
        if st != m.FLP_OK or st2 != m.FLP_OK:
            raise m.FlpError("flp_forward_indexed / flp_backward_indexed", st or st2)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    m.flp_profile_read()
    m.flp_profile_enable(True)
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    m.flp_profile_enable(False)
    prof = m.flp_profile_read()
    sel = int(torch.unique(ids[(ids >= 0) & (ids < N)]).numel())
    out = {"workload": f"{name} with {sel} of its {N} rows selected by {n_ids} ids (repeats, "
                       f"out-of-range ids): flp_forward_indexed + flp_backward_indexed",
           "N": N, "selected": sel, "ids": n_ids, "ms_per_step": round(ms, 4),
           "selected_tokens_per_s": round(sel / (ms / 1e3), 1),
           "row_kernels_ms_per_step": round(prof["rows"][0] / steps, 4),
           "method_TFLOPs": round(8.0 * min(n_ids, N) * D * V / (ms / 1e3) / 1e12, 1)}
    del prob, fws, bws, dh, dw
    return out


def embedding_op(N: int, D: int, V: int, steps: int, warmup: int):
    """The untied embedding lookup and its sorted-segment grad_weight at the model row's
    shape (HBM-bound: the lookup reads and writes N rows; the backward reads N gradient
    rows and writes all V rows of d_weight)."""
    import torch

    import flp_inputs
    import lm_head_selected_bf16_amd as m

    inp = flp_inputs.make_embedding_inputs(N, D, V, torch.bfloat16, 52, ids="zipf",
                                           device="cuda:0")
    w, g, ids = inp["weight"], inp["grad"], inp["ids"].cuda()
    out = torch.empty(N, D, dtype=torch.bfloat16, device="cuda:0")
    dw = torch.empty_like(w)
    ws = torch.empty(m.flp_embedding_backward_workspace_bytes(N, D, V), dtype=torch.uint8,
                     device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    fwd_ms, bwd_ms = [], []

    def call(timed):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record()
        st = m.flp_embedding_forward(N, D, V, m.FLP_BF16, w.data_ptr(), ids.data_ptr(),
                                     m.FLP_I64, out.data_ptr(), stream)
        e[1].record()
        st2 = m.flp_embedding_backward(N, D, V, m.FLP_BF16, g.data_ptr(), ids.data_ptr(),
                                       m.FLP_I64, dw.data_ptr(), m.FLP_BF16, ws.data_ptr(),
                                       ws.numel(), stream)
        e[2].record()
        if st != m.FLP_OK or st2 != m.FLP_OK:
            raise m.FlpError("flp_embedding_forward / flp_embedding_backward", st or st2)
        if timed:
            torch.cuda.synchronize()
            fwd_ms.append(e[0].elapsed_time(e[1]))
            bwd_ms.append(e[1].elapsed_time(e[2]))

    for _ in range(warmup):
        call(False)
    for _ in range(steps):
        call(True)
    f, b = sorted(fwd_ms)[len(fwd_ms) // 2], sorted(bwd_ms)[len(bwd_ms) // 2]
    fb = 2 * N * D * 2 + N * 8
    bb = N * D * 2 + V * D * 2 + N * 8
    res = {"workload": f"embedding_n{N}: untied bf16 table [{V}, {D}], zipf-drawn ids; lookup "
                       f"and sorted-segment d_weight (bf16, fp32 accumulation)",
           "distinct_ids": int(torch.unique(ids).numel())}
    for kind, ms, byts in (("forward", f, fb), ("backward", b, bb)):
        gbs = byts / (ms / 1e3) / 1e9
        res[kind] = {"ms": round(ms, 4), "bound": "hbm", "algorithmic_bytes": byts,
                     "achieved_GBs": round(gbs, 1), "peak_GBs": PEAK_HBM_GBS,
                     "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "frac_of_measured_peak": _meas_frac("hbm", gbs)}
    del w, g, out, dw, ws
    return res


def fwd_bwd(name: str, steps: int, warmup: int):
    """flp_forward + flp_backward on another workload (e.g. the 65600-token long sequence,
    whose backward runs in row chunks with the fp32 d_W accumulator continued across them)."""
    prob = Problem(name, backward=True)
    ms, _, prof = prob.time_steps(steps, warmup)
    N, D, V = prob.N, prob.D, prob.V
    fl = 8.0 * N * D * V
    out = {"workload": f"{name}: fwd+bwd, N={N}, D={D}, V={V}", "N": N, "steps": steps,
           "ms_per_step": round(ms, 3), "tokens_per_s": round(N / (ms / 1e3), 1),
           "method_TFLOPs": round(fl / (ms / 1e3) / 1e12, 1),
           "method_frac_of_peak": round(fl / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
           "backward_chunks": int(prof["dlogits"][1] // max(steps, 1)),
           "kernels_ms_per_step": {k: round(v[0] / steps, 3) for k, v in prof.items() if v[1]}}
    del prob
    return out


_MEAS = {}  # filled by measured_peaks(): the probes' achievable rates


def _meas_frac(bound: str, achieved: float):
    key = "stream_read_GBs" if bound == "hbm" else "mfma_bf16_random_operands_TFLOPs"
    return round(achieved / _MEAS[key], 4) if _MEAS.get(key) else None


def measured_peaks():
    """The chip's achievable rates from the library's probes: a dense bf16 MFMA loop on
    random and on zero operands (with the shader clock it ran at) and a streaming read of
    4 GiB."""
    import torch

    import lm_head_selected_bf16_amd as m

    sb = m.flp_probe_scratch_bytes()
    scratch = torch.empty(sb, dtype=torch.uint8, device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    out = {}
    for name, zero in (("random", False), ("zero", True)):
        st, tf, ghz = m.flp_probe_mfma(zero, 1000, scratch.data_ptr(), sb, stream)
        if st != m.FLP_OK:
            raise m.FlpError("flp_probe_mfma", st)
        out[f"mfma_bf16_{name}_operands_TFLOPs"] = round(tf, 1)
        out[f"clock_GHz_{name}_operands"] = round(ghz, 3)
    buf = torch.empty(4 << 30, dtype=torch.uint8, device="cuda:0")
    st, gbs = m.flp_probe_read(buf.data_ptr(), buf.numel(), scratch.data_ptr(), sb, stream)
    if st != m.FLP_OK:
        raise m.FlpError("flp_probe_read", st)
    out["stream_read_GBs"] = round(gbs, 1)
    _MEAS.update(out)
    out["note"] = ("flp_probe_mfma: 2048 workgroups x 4 waves of v_mfma_f32_16x16x32_bf16 on "
                   "register operands; flp_probe_read: 5 streaming passes over 4 GiB")
    del buf
    torch.cuda.empty_cache()
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the forward-only decode (N=32) and rollout (N=8192) figures")
    ap.add_argument("--only", choices=["decode_n32_forward", "rollout_n8192_forward"],
                    help="run just this forward-only figure and print its JSON (for profiling)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 3 times (reference for "
                         "the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": n}), flush=True)
        return 0
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    import torch
    import lm_head_selected_bf16_amd as m

    m.load()
    torch.cuda.set_device(0)
    if args.only:
        wl, bound = {"decode_n32_forward": ("decode_n32", "hbm"),
                     "rollout_n8192_forward": ("rollout_n8192", "mfma")}[args.only]
        print(json.dumps({args.only: forward_only(wl, args.steps, args.warmup, bound)}), flush=True)
        return 0
    log(m.flp_build_info())
    name = "train_n16384"
    log("measured peaks (probes)")
    peaks = measured_peaks()
    log(json.dumps(peaks))
    log(f"preparing {name}")
    prob = Problem(name, backward=True)
    N, D, V = prob.N, prob.D, prob.V
    log(f"warmup {args.warmup}, timing {args.steps} steps")
    ms, ems, prof = prob.time_steps(args.steps, args.warmup)
    log(f"{ms:.3f} ms/step (events {ems:.3f})")

    kernels = {}
    for kind, (tot, n) in prof.items():
        if n == 0:
            continue
        per_step = n / args.steps
        fl = contraction_flops(kind, N, D, V, int(round(per_step)))
        avg = tot / n
        kernels[kind] = {"ms_per_launch": round(avg, 4), "launches_per_step": per_step,
                         "ms_per_step": round(tot / args.steps, 4)}
        if fl:
            kernels[kind]["TFLOPs"] = round(fl / (avg / 1e3) / 1e12, 1)
    dom = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
    dom_n = int(round(kernels[dom]["launches_per_step"]))
    dom_fl = contraction_flops(dom, N, D, V, dom_n)
    dom_avg_s = kernels[dom]["ms_per_launch"] / 1e3
    achieved = dom_fl / dom_avg_s / 1e12
    meas = peaks["mfma_bf16_random_operands_TFLOPs"]
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 1),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": load_traffic(name, dom),
                "algorithmic_flops_per_launch": dom_fl,
                "measured_peak": meas, "frac_of_measured_peak": round(achieved / meas, 4)}
    step_flops = 8.0 * N * D * V
    value = N / (ms / 1e3)
    out = {
        "metric": "fwd+bwd tokens/s at D=2688,V=131072 bf16; % of MFMA / HBM roofline",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": round(value / PAGES_STRICT_TOK_S, 3),
        "baseline_note": "vs_baseline: over the pages' strict deterministic fwd+bwd at 16384 "
                         "tokens on H100 PCIe (351.2 ms), other hardware, context only; "
                         "vs_cpu_baseline: over the CPU FP64 oracle on this box's host cores "
                         "(cpu_baseline, the reported baseline)",
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "train_n16384: fwd+bwd, N=16384 tokens (B=4, S=4096), D=2688, "
                               "V=131072, bf16 hidden/W, fp32 bias, grad_out~N(0,1), bf16 d_W "
                               "with fp32 accumulation, single 16384-row backward chunk",
                   "N": N, "D": D, "V": V, "global_batch": 4, "seq_len": 4096,
                   "parallelism": "single GPU"},
        "ms_per_step_median": round(prob.step_ms_median, 4),
        "ms_per_step_min": round(prob.step_ms_min, 4),
        "method_TFLOPs": round(step_flops / (ms / 1e3) / 1e12, 1),
        "method_frac_of_peak": round(step_flops / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "method_frac_of_measured_peak": round(step_flops / (ms / 1e3) / 1e12 / meas, 4),
        "measured_peaks": peaks,
        "provenance": {"build_info": m.flp_build_info(), "fallback": False,
                       "library": os.path.relpath(m._abi.LIB_PATH, ROOT)},
        "roofline": roofline,
        "kernels": kernels,
    }
    del prob
    torch.cuda.empty_cache()
    if not args.no_extra:
        log("forward-only: decode_n32")
        out["decode_n32_forward"] = forward_only("decode_n32", 50, 10, "hbm")
        log("forward-only: rollout_n8192")
        out["rollout_n8192_forward"] = forward_only("rollout_n8192", 10, 3, "mfma")
        log("one vocabulary shard of 8: decode_n32, rollout_n8192")
        out["decode_n32_shard8_forward"] = shard_forward("decode_n32", 8, 50, 10, "hbm")
        out["rollout_n8192_shard8_forward"] = shard_forward("rollout_n8192", 8, 10, 3, "mfma")
        torch.cuda.empty_cache()
        log("operator on materialised logits: N=8192, V=131072")
        out["logits_op_n8192"] = logits_op(8192, 131072, 10, 3)
        torch.cuda.empty_cache()
        log("indexed: half of train_n16384's rows")
        out["train_n16384_indexed_half"] = indexed_step(name, N // 2, 5, 2)
        torch.cuda.empty_cache()
        log("untied embedding lookup: N=16384, D=2688, V=131072")
        out["embedding_n16384"] = embedding_op(16384, 2688, 131072, 10, 3)
        torch.cuda.empty_cache()
        log("long sequence: longseq_n65600 fwd+bwd")
        out["longseq_n65600_fwd_bwd"] = fwd_bwd("longseq_n65600", 2, 1)
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        cpu_prob = Problem.__new__(Problem)
        import flp_inputs
        cpu_prob.cpu = flp_inputs.make_inputs(name)
        cpu_prob.w = cpu_prob.cpu["workload"]
        cpu_prob.N, cpu_prob.D, cpu_prob.V = cpu_prob.w.N, cpu_prob.w.D, cpu_prob.w.V
        out["cpu_baseline"] = cpu_baseline(cpu_prob)
        out["vs_cpu_baseline"] = round(out["value"] / out["cpu_baseline"]["value"], 1)
        out["cpu_oracle_configs"] = cpu_oracle_configs()
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
