"""The fp64 oracle against closed forms, identities, library routines and laws."""
from tests import oracle_pins as pins


def test_closed_form_features():
    pins.check_closed_form_features()


def test_closed_form_attention():
    pins.check_closed_form_attention()


def test_associative_vs_explicit():
    pins.check_associative_vs_explicit()


def test_causal_scan_vs_quadratic():
    pins.check_causal_vs_quadratic()


def test_performer_special_case():
    pins.check_performer_special_case()


def test_mc_kernel_estimate():
    pins.check_mc_kernel()


def test_output_converges_to_exact():
    pins.check_output_convergence()


def test_exact_limit_vs_sdpa():
    pins.check_exact_vs_sdpa()


def test_invariants():
    pins.check_invariants()


def test_scaling_rule():
    pins.check_scaling_rule()


def test_decode_recurrence_vs_causal():
    pins.check_decode_vs_causal()


def test_context_state_explicit():
    pins.check_context_state_explicit()


def test_cross_vs_explicit():
    pins.check_cross_vs_explicit()


def test_backward_finite_differences():
    pins.check_backward_finite_differences()


def test_backward_linear_form():
    pins.check_backward_linear_form()


def test_per_head_projection():
    pins.check_per_head_projection()
