"""The measurement probes (flp_probe_mfma, flp_probe_read) run and return rates
within physical bounds for one MI355X: below the nominal 2.5 PFLOP/s dense bf16
and 8 TB/s, and far above what a broken probe would give."""
import pytest
import torch

from gpu_common import flp, say

pytestmark = pytest.mark.gpu


def test_probes_in_physical_range():
    m = flp()
    sb = m.flp_probe_scratch_bytes()
    scratch = torch.empty(sb, dtype=torch.uint8, device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    st, tf_r, ghz_r = m.flp_probe_mfma(False, 200, scratch.data_ptr(), sb, stream)
    assert st == m.FLP_OK
    st, tf_z, ghz_z = m.flp_probe_mfma(True, 200, scratch.data_ptr(), sb, stream)
    assert st == m.FLP_OK
    buf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0")
    st, gbs = m.flp_probe_read(buf.data_ptr(), buf.numel(), scratch.data_ptr(), sb, stream)
    assert st == m.FLP_OK
    say(f"mfma random {tf_r:.0f} TF at {ghz_r:.2f} GHz, zero {tf_z:.0f} TF at {ghz_z:.2f} GHz, "
        f"read {gbs:.0f} GB/s")
    assert 500 < tf_r <= 2600 and 500 < tf_z <= 2600
    assert 0.8 < ghz_r < 3.0 and 0.8 < ghz_z < 3.0
    assert 1000 < gbs < 8500
