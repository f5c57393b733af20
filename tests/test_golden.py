"""The oracle against its stored regression record (tests/golden)."""
import json
import os

import numpy as np

from golden.make_golden import record

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_tiny_layer_matches_stored_oracle_record():
    want = json.load(open(os.path.join(HERE, "tiny_layer_oracle.json")))
    got = record()
    assert got["ids"] == want["ids"]
    for k in ("scores", "logits", "out_first16"):
        np.testing.assert_allclose(got[k], want[k], rtol=1e-12, atol=1e-12)
    for k in ("out_sum", "act_sum"):
        assert abs(got[k] - want[k]) <= 1e-10 * max(1.0, abs(want[k]))
