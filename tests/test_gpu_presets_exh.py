"""The exhaustive preset (80M items, d = 64, nprobe = nlist): a pure streaming filter + score +
select pass.  Sampled oracle parity, invariants on every query."""
import numpy as np
import pytest

from test_gpu_presets import Preset, svt  # noqa: F401  (module fixture)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pexh(svt):  # noqa: F811
    p = Preset(svt, "exh")
    yield p
    p.close()


def test_exhaustive_batch32(pexh):
    pexh.check(32, 0, sample=[0, 13, 31], label="exh-b32")
