"""The oracle against what the pages and the mathematics fix (CPU only)."""
import pytest

import oracle.verify as vm
from tests import oracle_pins as pins


def test_abr_worked_example():
    pins.pin_abr_example(vm)


def test_weather_greedy_example():
    pins.pin_weather_example(vm)


def test_t1_t4_round():
    pins.pin_t1_t4_round(vm)


def test_greedy_tie_reading():
    pins.pin_greedy_ties(vm)


def test_exact_distribution_by_quadrature():
    pins.pin_exact_distribution_quadrature(vm)


def test_monte_carlo_distribution_and_acceptance():
    pins.pin_monte_carlo(vm)


def test_special_cases():
    pins.pin_special_cases(vm)


def test_greedy_invariants():
    pins.pin_greedy_invariants(vm)


def test_cost_model_illustration():
    pins.pin_cost_model()


def test_decision_margins():
    pins.pin_decision_margins(vm)


def test_temperature_reading():
    pins.pin_temperature_reading(vm)


def test_early_exit_form():
    pins.pin_early_exit_form(vm)


def test_packed_ragged_batch():
    pins.pin_packed_batch(vm)


def test_invalid_stochastic_token_rejected():
    import numpy as np
    z = np.zeros((2, 5))
    with pytest.raises(ValueError):
        vm.verify_request(z, z[:1], np.array([7]), False, 1.0, np.array([0.5]), 0.5)
