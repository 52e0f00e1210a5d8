"""The oracle still reproduces its frozen regression fixture."""
import json
import os

import numpy as np

from tests.golden.make_golden import OUT, compute


def test_oracle_matches_frozen_fixture():
    with open(OUT) as f:
        want = json.load(f)
    got = json.loads(json.dumps(compute()))
    assert got["seq_lens"] == want["seq_lens"]
    assert got["planted"] == want["planted"]
    assert got["selected"] == want["selected"]
    for key in ("verify_o_first4", "verify_lse", "sparse_o_first4", "sparse_lse", "scores"):
        for name, val in want[key].items():
            np.testing.assert_allclose(got[key][name], val, rtol=0, atol=1e-12, err_msg=f"{key}[{name}]")
