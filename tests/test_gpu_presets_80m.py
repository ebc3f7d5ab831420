"""The 80M-item presets (d = 128 IVF, and d = 64 exhaustive) at full size: sampled oracle parity in
the launch configuration the benchmark times, invariants on every query."""
import numpy as np
import pytest

from test_gpu_presets import Preset, svt  # noqa: F401  (module fixture)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def p80(svt):  # noqa: F811
    p = Preset(svt, "80m")
    yield p
    p.close()


def test_80m_batch256(p80):
    p80.check(256, 0, sample=np.arange(0, 256, 16), label="80m-b256")


def test_80m_batch32(p80):
    p80.check(32, 20_000, sample=np.arange(0, 32, 4), label="80m-b32")


def test_80m_batch1(p80):
    for off in (40_000, 40_001, 40_002):
        p80.check(1, off, label=f"80m-b1-{off}")
