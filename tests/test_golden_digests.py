"""The oracle's masks still match the stored digests (written from oracle/ only)."""

import os

from tests.golden.gen_mask_digests import lines

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_oracle_masks_match_stored_digests():
    with open(os.path.join(HERE, "mask_digests.txt")) as f:
        stored = [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]
    assert stored == lines()
