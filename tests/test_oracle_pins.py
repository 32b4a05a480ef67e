"""The fp64 oracle against the pages' printed values, closed forms, brute
force and library routines (CPU only)."""
import pytest

import oracle_pins as P


@pytest.mark.parametrize("check", P.ALL, ids=lambda f: f.__name__)
def test_pin(check):
    check()


def test_brute_force_square_no_shared():
    P.check_brute_force(seed=11, T=16, d=12, E=5, k=2, n_shared=0, square=True)


def test_brute_force_k_equals_E():
    P.check_brute_force(seed=12, T=10, d=8, E=4, k=4, n_shared=2)
