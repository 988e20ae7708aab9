"""Pins of the oracle's OMP comparison encoder (oracle.omp_encode): agreement
with the pursuit where the refit changes nothing (orthonormal dictionary,
K = 1), the defining properties of the least-squares refit, exact recovery
of a coherent support that the pursuit alone cannot finish, exact
rational brute force on tiny integer inputs, and the exact-fit case (a
residual that reaches zero)."""
import oracle
from tests import oracle_pins as pins


def test_omp_equals_mp_where_the_refit_is_a_projection():
    pins.check_omp_equals_mp_on_orthonormal(oracle.omp_encode, oracle.mp_encode)


def test_omp_refit_properties():
    pins.check_omp_refit_properties(oracle.omp_encode)


def test_omp_exact_recovery_of_a_coherent_support():
    pins.check_omp_exact_recovery_coherent_support(oracle.omp_encode, oracle.mp_encode)


def test_omp_rational_bruteforce():
    pins.check_omp_bruteforce_rational(oracle.omp_encode)


def test_omp_exact_fit():
    pins.check_omp_exact_fit(oracle.omp_encode)
