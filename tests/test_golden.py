"""The oracle's bit-exact outputs still hash to the committed golden values."""
import json
import os
import sys

import pytest

sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden"))
import make_hashes  # noqa: E402

GOLDEN = json.load(open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hashes.json")))


@pytest.mark.parametrize("name", ["c0", "c1", "c2", "c3", "c4"])
def test_oracle_hashes(name):
    got = {k: make_hashes.sha(v) for k, v in make_hashes.bit_exact_outputs(name).items()}
    assert got == GOLDEN[name]
