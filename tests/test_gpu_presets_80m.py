"""The 80M-item IVF preset (d = 128, nlist 16384, nprobe 64, top-2048) at full size, in the launch
configuration the benchmark times: every query of every batch compared with the oracle, on both search
paths, plus the size-independent invariants."""
import pytest

from test_gpu_presets import Preset, svt  # noqa: F401  (module fixture)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def p80(svt):  # noqa: F811
    p = Preset(svt, "80m")
    yield p
    p.close()


def test_80m_batch256(p80):
    p80.check(256, 0, label="80m-b256")


def test_80m_batch32(p80):
    p80.check(32, 20_000, label="80m-b32")


def test_80m_batch1(p80):
    for off in (40_000, 40_001, 40_002):
        p80.check(1, off, label=f"80m-b1-{off}")
