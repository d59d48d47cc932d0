"""attn_clock_probe on an idle GPU: the wave waits until the 100 MHz
real-time counter has advanced by spin_us * 100 ticks (one sleep-and-read
step of overshoot at most) and reports the shader cycles it counted meanwhile,
which give the clock the bench line quotes."""
import pytest
import torch

from exact_attention_forward_06_amd import clock_probe

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("spin_us", [50, 300])
def test_clock_probe_idle(spin_us):
    out = clock_probe(spin_us)
    torch.cuda.synchronize()
    cycles, ticks = (int(x) for x in out.cpu())
    want = spin_us * 100
    assert want <= ticks <= want + max(100, want // 20), (ticks, want)
    mhz = cycles / ticks * 100
    assert 300.0 <= mhz <= 3000.0, mhz
