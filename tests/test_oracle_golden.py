"""The oracle still reproduces the fixtures written by tests/golden/make_golden.py."""
import json
import os

import numpy as np
import pytest

from oracle import vx_oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.mark.parametrize("name", ["hand_example", "seeded_small"])
def test_oracle_matches_fixture(name):
    with open(os.path.join(GOLDEN, name + ".json")) as f:
        case = json.load(f)
    seq = {"q": np.array(case["q"]), "k": np.array(case["k"]), "v": np.array(case["v"]),
           "seq_len": case["seq_len"],
           "rand_u32": np.zeros(case["params"]["num_kv_heads"], np.uint32)}
    r = O.decode_sequence(seq, **case["params"])
    for key, want in case["expect"].items():
        np.testing.assert_allclose(np.asarray(r[key], dtype=np.float64),
                                   np.asarray(want, dtype=np.float64), rtol=1e-12, atol=1e-12)
