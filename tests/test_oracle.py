"""The CPU oracle against its pins (no GPU)."""
import pytest

import oracle
import oracle_pins as P


@pytest.fixture(scope="module")
def orc():
    return oracle.Oracle()


def test_splitmix64_published(orc):
    P.pin_splitmix64(orc)


def test_handworked_example(orc):
    P.pin_handworked(orc)


@pytest.mark.parametrize("W", [1, 2])
@pytest.mark.parametrize("d", [16, 32, 64])
def test_exhaustive_equals_library_topk(orc, W, d):
    P.pin_exhaustive(orc, seed=10 + d + W, W=W, d=d)


def test_exhaustive_tie_heavy(orc):
    P.pin_exhaustive(orc, seed=11, tie_heavy=True, d=16, k=200)


def test_probe_set_order(orc):
    P.pin_probe_set(orc)


def test_ivf_is_restricted_exhaustive(orc):
    P.pin_ivf_restriction(orc)


def test_mask_groups(orc):
    P.pin_mask_groups(orc)


def test_padding(orc):
    P.pin_padding(orc)


def test_dequant_exact_rational(orc):
    P.pin_dequant(orc)


def test_bloom_closed_form_and_no_false_negatives(orc):
    P.pin_bloom(orc)


def test_bloom_mapping_golden(orc):
    P.pin_bloom_mapping(orc)


def test_mask_helper(orc):
    P.pin_mask_helper(orc)


def test_bloom_closed_form_values():
    # the exact closed form evaluated for the two signature shapes used by the presets
    assert abs(float(P.bloom_fp_exact(64, 3, 2)) - 0.008180) < 5e-7
    assert abs(float(P.bloom_fp_exact(128, 5, 3)) - 0.001381) < 5e-7
