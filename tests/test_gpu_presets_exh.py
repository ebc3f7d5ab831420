"""The exhaustive preset (80M items, d = 64, nprobe = nlist): one streaming filter + score + select pass
over the whole catalogue per batch.  Every query compared with the oracle on both search paths (query by
query, and the int8 MFMA scan that reads the catalogue once for the batch), plus the invariants."""
import pytest

from test_gpu_presets import Preset, svt  # noqa: F401  (module fixture)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pexh(svt):  # noqa: F811
    p = Preset(svt, "exh")
    yield p
    p.close()


def test_exhaustive_batch32(pexh):
    pexh.check(32, 0, label="exh-b32")


def test_exhaustive_batch4(pexh):
    pexh.check(4, 100, label="exh-b4")
