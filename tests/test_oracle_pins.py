"""The fp64 oracle against what the pages and the mathematics fix (CPU only)."""
import pytest

from oracle import paged_ref
from tests import oracle_checks as oc


@pytest.mark.parametrize("check", oc.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check(paged_ref)
