"""The oracle against what the pages and mathematics fix (CPU only)."""
import pytest

import oracle.calculator as calc
import oracle.verify as ov
import oracle_pins as pins


@pytest.mark.parametrize("pin", pins.ALL_ORACLE_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(ov)


@pytest.mark.parametrize("setting", pins.SETTINGS, ids=lambda s: "T%g-k%d-p%g" % (s["T"], s["top_k"], s["top_p"]))
def test_chisq_emitted_tokens(setting):
    pins.pin_chisq(ov, setting=setting)


def test_constant_alpha_matches_calculator():
    pins.pin_constant_alpha(ov, calc)


def test_calculator():
    pins.pin_calculator(calc)


import oracle.aux as ax


def test_aux_golden():
    pins.pin_aux_golden(ax)


def test_tree_mask_recursion():
    pins.pin_mask_recursion(ax)


def test_commit_map_inverts_the_path():
    pins.pin_commit_inverse(ax)


def test_measured_alpha_recovers_the_model():
    pins.pin_alpha_recovery(ax, calc)


import oracle.tree_sample as ts


def test_tree_sample_golden():
    pins.pin_tree_sample_golden(ts)


def test_tree_sample_path_is_chain():
    pins.pin_tree_sample_is_chain(ts, ov)


def test_tree_sample_enumeration():
    pins.pin_tree_sample_enumeration(ts, ov)


def test_tree_sample_chisq():
    pins.pin_tree_sample_chisq(ts, ov)


def test_tree_sample_status():
    pins.pin_tree_sample_status(ts)


def test_tree_sample_flags():
    pins.pin_tree_sample_flags(ts)
