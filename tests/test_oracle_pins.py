"""The CPU oracle against the pages' worked example, invariants, closed forms
and finite differences (no GPU)."""

import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_FORWARD_PINS, ids=lambda f: f.__name__)
def test_forward_pin(pin):
    pin()


def test_bwd_finite_differences_single_head_per_destination_gain():
    pins.pin_bwd_finite_differences(1, "per")


def test_bwd_finite_differences_two_heads_shared_gain():
    pins.pin_bwd_finite_differences(2, "shared")


def test_bwd_finite_differences_no_gain_eps_zero():
    pins.pin_bwd_finite_differences(1, None, eps=0.0)


def test_bwd_closed_forms():
    pins.pin_bwd_closed_forms()


@pytest.mark.parametrize("H,gain,n_dst", [(1, "per", 5), (2, "shared", 3), (1, None, 2), (4, "per", 5)])
def test_full_bwd_finite_differences(H, gain, n_dst):
    pins.pin_full_bwd_finite_differences(H, gain, n_dst)


def test_full_bwd_finite_differences_eps_zero():
    pins.pin_full_bwd_finite_differences(1, "per", 4, eps=0.0)


def test_full_bwd_single_source():
    pins.pin_full_bwd_single_source()


def test_full_bwd_block_s1_identity():
    pins.pin_full_bwd_block_s1_identity()


def test_tolerance_metric():
    pins.pin_tolerance_error()
