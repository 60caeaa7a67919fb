"""Vocabulary shards ("Fused Linear LogP" docs page, "Tensor Parallel Vocab
Shards"): the weight split into row ranges on 256-column tile boundaries, one
flp_forward_partial per shard, the partials concatenated in vocabulary order and
the shards' zt added, then flp_merge.  Every tile partial of a shard equals the
unsharded one and the merge folds them in the same order, so logp and lse must
equal the unsharded flp_forward bit for bit; they are also held to the oracle."""
import numpy as np
import pytest
import torch

import flp_inputs
from gpu_common import LOGP_CELL, check_close, flp, gpu_forward, inputs, oracle_forward, say, to_gpu

pytestmark = pytest.mark.gpu
BF16 = torch.bfloat16


def sharded_forward(g, bounds):
    """logp, lse of the shards [bounds[k], bounds[k + 1])."""
    m = flp()
    V = int(g["weight"].shape[0])
    parts, zt = [], None
    for lo, hi in zip(bounds[:-1], bounds[1:]):
        b = None if g["bias"] is None else g["bias"][lo:hi].contiguous()
        p, z = m.forward_partial(g["hidden"], g["weight"][lo:hi].contiguous(), g["targets"], lo, V,
                                 bias_shard=b, temperature=g["temperature"])
        parts.append(p)
        zt = z if zt is None else zt + z
    return m.merge(torch.cat(parts, dim=0).contiguous(), zt, g["targets"], V)


def small_case(N, D, V, seed, t_dtype=torch.int64):
    w = flp_inputs.Workload(f"shards{seed}", 200 + seed, N, D, V, BF16, w_std=1.3 / np.sqrt(D),
                            bias_std=0.1, n_ignored=5, ignore_values=(-1, V, -100, V + 7),
                            temperature=(0.5, 1.5), grad="ones", leading=(N,))
    inp = flp_inputs.make_inputs(w)
    inp["targets"] = inp["targets"].to(t_dtype)
    return inp


@pytest.mark.parametrize("bounds_fn,t_dtype", [
    (lambda V: [0, V], torch.int64),                      # one shard: the whole vocabulary
    (lambda V: [0, 256, 1024, V], torch.int64),           # uneven shards, ragged last tile
    (lambda V: [0, 512, 768, 1280, V], torch.int32),
])
def test_shards_small_bitwise(bounds_fn, t_dtype):
    N, D, V = 300, 256, 1300
    inp = small_case(N, D, V, 1, t_dtype)
    g = to_gpu(inp)
    bounds = bounds_fn(V)
    say(f"shards {bounds} N={N} D={D} V={V} targets {t_dtype}")
    lp, ls = sharded_forward(g, bounds)
    lp0, ls0 = gpu_forward(g)
    torch.cuda.synchronize()
    assert torch.equal(lp, lp0) and torch.equal(ls, ls0)
    ref_lp, ref_ls = oracle_forward(inp)
    check_close("logp", lp, ref_lp, **LOGP_CELL)
    check_close("lse", ls, ref_ls, **LOGP_CELL)


def test_shards_decode_tp8_bitwise():
    """The decode workload (N=32, D=2688, V=131072) split as an 8-way vocabulary
    tensor-parallel head would be: 8 shards of 16384 rows."""
    inp = inputs("decode_n32")
    g = to_gpu(inp)
    V = int(g["weight"].shape[0])
    bounds = list(range(0, V + 1, V // 8))
    say(f"decode_n32, shards of {V // 8}")
    lp, ls = sharded_forward(g, bounds)
    lp0, ls0 = gpu_forward(g)
    torch.cuda.synchronize()
    assert torch.equal(lp, lp0) and torch.equal(ls, ls0)
    ref_lp, ref_ls = oracle_forward(inp)
    check_close("logp", lp, ref_lp, **LOGP_CELL)
    check_close("lse", ls, ref_ls, **LOGP_CELL)


def test_shard_zt_is_zero_outside_the_shard():
    inp = small_case(64, 128, 1024, 2)
    g = to_gpu(inp)
    m = flp()
    _, zt = m.forward_partial(g["hidden"], g["weight"][256:768].contiguous(), g["targets"], 256,
                              1024, bias_shard=g["bias"][256:768].contiguous(),
                              temperature=g["temperature"])
    t = inp["targets"].numpy()
    outside = ~((t >= 256) & (t < 768))
    assert np.all(zt.cpu().numpy()[outside] == 0.0)


def test_shard_rejects_misaligned_start():
    inp = small_case(16, 64, 1000, 3)
    g = to_gpu(inp)
    m = flp()
    with pytest.raises(m.FlpError, match="UNSUPPORTED_SHAPE"):
        m.forward_partial(g["hidden"], g["weight"][100:612].contiguous(), g["targets"], 100, 1000)
