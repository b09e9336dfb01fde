"""The oracle still reproduces its stored golden fixtures.

The fixtures under ``tests/golden/`` were written by
``tests/golden/make_golden.py``, which calls only the oracle. A change to
the oracle's arithmetic fails here until the fixtures are rewritten.
"""

import json
import os

import numpy as np
import pytest

from tests.golden import make_golden

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.mark.parametrize("name", sorted(make_golden.CASES))
def test_oracle_reproduces_golden(name):
    with open(os.path.join(HERE, f"{name}.json")) as f:
        stored = json.load(f)["values"]
    now = make_golden.run_case(make_golden.CASES[name])
    assert set(now) == set(stored)
    for k, v in stored.items():
        np.testing.assert_allclose(np.asarray(now[k]), np.asarray(v), rtol=1e-12,
                                   atol=1e-15, err_msg=k)
