"""The synthetic quality study (tests/quality_study.py), on the CPU oracle:
the Hermitian-unpack real-DFT variant pinned to its definition, and the
study's measured facts checked on 8192 vectors per law."""

import math

import numpy as np
import pytest

import oracle as O
from tests import quality_study as Q


@pytest.mark.parametrize("D", [2, 4, 8, 16])
def test_hermitian_variant_equals_basis_matrix(D):
    """The real-DFT variant against its cosine / sine basis built in pure
    Python (no FFT), for random signs."""
    s = (1 - 2 * np.random.default_rng(D).integers(0, 2, D)).astype(np.int8)
    R = O.rotation_matrix(D, O.HERMITIAN, s)
    Rb = np.array(O.hermitian_matrix_bruteforce(D, [int(v) for v in s]))
    assert np.max(np.abs(R - Rb)) < 1e-12


@pytest.mark.parametrize("D", [8, 128, 256])
def test_hermitian_variant_orthogonal_and_inverse(D):
    s = O.plan_signs(D, O.HERMITIAN, 11)
    assert s.size == D
    R = O.rotation_matrix(D, O.HERMITIAN, s)
    assert np.max(np.abs(R @ R.T - np.eye(D))) < 1e-12
    x = np.random.default_rng(2).standard_normal((5, D))
    assert np.max(np.abs(O.rotate_inverse(O.rotate_forward(x, O.HERMITIAN, s), O.HERMITIAN, s) - x)) < 1e-12
    # a constant signed vector lands entirely in the DC coordinate
    y = O.rotate_forward(s.astype(np.float64)[None, :], O.HERMITIAN, s)[0]
    assert abs(y[0] - math.sqrt(D)) < 1e-12 and np.max(np.abs(y[1:])) < 1e-12


@pytest.fixture(scope="module")
def study():
    return Q.table(8192)


def test_study_per_token_fails_on_outliers(study):
    """One scale per vector without rotation is several times worse than the
    rotated per-group quantizer on every law."""
    for key, r in study.items():
        assert r["per-token int4 (no rotation)"] > 4 * r["SRFT G32 int4"], key
        assert r["per-token int4 (no rotation)"] > 4 * r["SRHT G32 int4"], key


def test_study_srht_never_worse_than_no_rotation(study):
    for key, r in study.items():
        assert r["SRHT G32 int4"] < r["per-group G32 int4 (no rotation)"], key


def test_study_srft_and_srht_close_at_d128(study):
    """SRFT within 10% of SRHT at D=128 on both laws.  (At D=256 on the
    channel-spread law SRFT is about twice SRHT: a dominant channel gives the
    SRFT output cos^2 / sin^2-shaped variances across frequencies, while the
    +-1 entries of the Hadamard matrix spread any diagonal covariance evenly.)"""
    for key in (("spread", 128), ("t3", 128)):
        r = study[key]
        assert abs(r["SRFT G32 int4"] / r["SRHT G32 int4"] - 1) < 0.10, key
    r = study[("spread", 256)]
    assert r["SRFT G32 int4"] > 1.5 * r["SRHT G32 int4"]


def test_study_hermitian_variant_tracks_srft(study):
    for key, r in study.items():
        assert abs(r["real-DFT (Hermitian unpack) G32 int4"] / r["SRFT G32 int4"] - 1) < 0.05, key


def test_study_finer_groups_and_wider_codes_help(study):
    for key, r in study.items():
        assert r["SRFT G16 int4"] < r["SRFT G32 int4"], key
        assert r["SRHT G16 int4"] < r["SRHT G32 int4"], key
        # int8 against int4: the step shrinks 127/7-fold, the error ~330-fold
        assert r["SRFT G32 int8"] < r["SRFT G32 int4"] / 100, key
        assert r["SRHT G32 int8"] < r["SRHT G32 int4"] / 100, key
