"""Closed forms and invariants of the operator, checked on the HIP path itself
(through the C ABI) rather than against the oracle: the same properties that pin
the oracle (its test file) must hold for the GPU results.

- Normalisation: one hidden row replicated V times with targets 0 .. V-1 gives
  log-probabilities whose exponentials sum to 1, and every replica has the same
  LSE bits (a row's results do not depend on the other rows).
- W = 0 and b = 0: every logit is 0, so lse = log V and logp = -log V.
- Adding a constant to every bias entry leaves logp unchanged and shifts lse.
- The gradients are linear in grad_out: scaling it by 2 is exact in every
  floating-point format here, so the gradients double bit for bit; grad_out = 0
  gives exactly zero gradients.
- A power-of-two temperature equals scaling W and b, bit for bit (the temperature
  divides the whole logit).
- A row's LSE does not depend on its target."""
import math

import numpy as np
import pytest
import torch

import flp_inputs
from gpu_common import gpu_backward, gpu_forward, say, to_gpu

pytestmark = pytest.mark.gpu

BF16 = torch.bfloat16


def _inputs(dtype, N=96, D=256, V=4096, bias_std=0.1, temperature=(0.5, 1.5), seed=401):
    w = flp_inputs.Workload(f"props{seed}", seed, N, D, V, dtype, w_std=0.05, bias_std=bias_std,
                            n_ignored=3, ignore_values=(-1, V), temperature=temperature,
                            grad="normal", leading=(N,))
    return flp_inputs.make_inputs(w)


@pytest.mark.parametrize("dtype", [torch.float32, BF16])
def test_replicated_row_normalisation(dtype):
    """sum_v exp(logp(h, t = v)) = 1 for one row replicated over every target."""
    inp = _inputs(dtype)
    V = inp["workload"].V
    say(f"case normalisation: D=256 V={V} {dtype}, one row x {V} targets")
    g = to_gpu(inp)
    rep = dict(g)
    rep["hidden"] = g["hidden"][5:6].expand(V, -1).contiguous()
    rep["targets"] = torch.arange(V, device="cuda:0", dtype=torch.int64)
    rep["temperature"] = g["temperature"][5:6].expand(V).contiguous()
    logp, lse = gpu_forward(rep)
    total = float(torch.exp(logp.double()).sum())
    say(f"  sum exp(logp) - 1 = {total - 1.0:.3e}")
    assert abs(total - 1.0) < 1e-5
    assert torch.equal(lse, lse[:1].expand(V))


@pytest.mark.parametrize("dtype", [torch.float32, BF16])
def test_zero_weight_gives_uniform(dtype):
    """W = 0, b = 0: lse = log V and logp = -log V for every valid target, any T."""
    inp = _inputs(dtype, V=1000)
    g = to_gpu(inp)
    g["weight"] = torch.zeros_like(g["weight"])
    g["bias"] = torch.zeros_like(g["bias"])
    V = inp["workload"].V
    say(f"case zero weight: V={V} {dtype}")
    logp, lse = gpu_forward(g)
    t = g["targets"]
    valid = (t >= 0) & (t < V)
    assert torch.allclose(lse.double(), torch.full_like(lse.double(), math.log(V)), rtol=0, atol=1e-6)
    assert torch.allclose(logp[valid].double(), torch.full_like(logp[valid].double(), -math.log(V)),
                          rtol=0, atol=1e-6)
    assert torch.all(logp[~valid] == 0.0)


@pytest.mark.parametrize("dtype", [torch.float32, BF16])
def test_bias_shift(dtype):
    """b + c leaves logp unchanged and shifts lse by c / T (up to fp32 rounding of the
    shifted logits)."""
    inp = _inputs(dtype)
    g = to_gpu(inp)
    c = 3.0
    logp0, lse0 = gpu_forward(g)
    g2 = dict(g)
    g2["bias"] = g["bias"] + c
    logp1, lse1 = gpu_forward(g2)
    T = g["temperature"].double()
    say(f"case bias shift: {dtype}, c = {c}")
    assert torch.allclose(logp1.double(), logp0.double(), rtol=0, atol=2e-5)
    assert torch.allclose(lse1.double() - lse0.double(), c / T, rtol=0, atol=2e-5)


@pytest.mark.parametrize("dtype", [torch.float32, BF16])
def test_gradients_linear_in_grad_out(dtype):
    """2 grad_out gives exactly twice every gradient; grad_out = 0 gives exact zeros."""
    inp = _inputs(dtype)
    g = to_gpu(inp)
    _, lse = gpu_forward(g)
    say(f"case gradient linearity: {dtype}")
    dh1, dw1, db1 = gpu_backward(g, lse, need_bias=True)
    dh2, dw2, db2 = gpu_backward(g, lse, grad_out=2.0 * g["grad_out"], need_bias=True)
    assert torch.equal(dh2, 2 * dh1)
    assert torch.equal(dw2, 2 * dw1)
    assert torch.equal(db2, 2 * db1)
    dh0, dw0, db0 = gpu_backward(g, lse, grad_out=torch.zeros_like(g["grad_out"]), need_bias=True)
    assert not torch.any(dh0 != 0) and not torch.any(dw0 != 0) and not torch.any(db0 != 0)
    # every valid row's dz sums to zero over the vocabulary, so d_bias sums to ~0
    scale = float(db1.abs().sum())
    assert abs(float(db1.double().sum())) <= 1e-4 * max(scale, 1.0)
    np.testing.assert_array_equal(np.isfinite(dh1.float().cpu().numpy()), True)


@pytest.mark.parametrize("dtype", [torch.float32, BF16])
def test_power_of_two_temperature_scales_the_whole_logit(dtype):
    """T = 2^k: dividing (h W^T + b) by T equals scaling W and b by 2^-k, bit for bit,
    because a power-of-two scaling commutes with every rounding (no value here comes
    near the under- or overflow range).  This pins the reading that the temperature
    divides the whole logit, bias included."""
    inp = _inputs(dtype, temperature=None)
    g = to_gpu(inp)
    N = inp["workload"].N
    k = 2
    g1 = dict(g)
    g1["temperature"] = torch.full((N,), float(2 ** k), device="cuda:0")
    g2 = dict(g)
    g2["weight"] = g["weight"] * (2.0 ** -k)
    g2["bias"] = g["bias"] * (2.0 ** -k)
    say(f"case temperature 2^{k}: {dtype}")
    logp1, lse1 = gpu_forward(g1)
    logp2, lse2 = gpu_forward(g2)
    assert torch.equal(logp1, logp2)
    assert torch.equal(lse1, lse2)


@pytest.mark.parametrize("dtype", [torch.float32, BF16])
def test_lse_does_not_depend_on_the_target(dtype):
    """A row's LSE is the same bits whatever its target, ignored targets included."""
    inp = _inputs(dtype)
    g = to_gpu(inp)
    V = inp["workload"].V
    _, lse0 = gpu_forward(g)
    g2 = dict(g)
    t = g["targets"].clone()
    t[::2] = (t[::2] + 1234) % V
    t[1::7] = -100
    t[3::11] = V + 5
    g2["targets"] = t
    say(f"case lse vs target: {dtype}")
    _, lse1 = gpu_forward(g2)
    assert torch.equal(lse0, lse1)
