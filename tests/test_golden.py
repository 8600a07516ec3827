"""The oracle's tiny-layer intermediates must not drift from the committed
digests (tests/golden/tiny_oracle.json, written by tests/golden/make_golden.py).
A deliberate change to the oracle's arithmetic regenerates the file and names
the passage that justifies it in its commit message."""
import json
import os

from tests.golden.make_golden import tiny_record


def test_tiny_oracle_digests_unchanged():
    path = os.path.join(os.path.dirname(__file__), "golden", "tiny_oracle.json")
    want = json.load(open(path))
    got = tiny_record()
    for k, v in got.items():
        assert want[k] == v, k
