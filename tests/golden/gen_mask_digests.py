"""Write tests/golden/mask_digests.txt from the oracle (and only the oracle).

One line per (workload shape, rotation flag, step): the SHA-256 of the CSR
mask as little-endian int32 (row_ptr then col_idx).  Locks the oracle's mask
so that any later change to its arithmetic shows up in review.

    python tests/golden/gen_mask_digests.py
"""

import hashlib
import os
import struct
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle.mask as om  # noqa: E402

SHAPES = [  # (name, T, C, W, steps)
    ("tiny", 8, 4, 2, 8),
    ("wan13b_1x", 21, 21, 9, 50),
    ("wan_6x", 121, 21, 9, 50),
    ("syn_1p5x", 49, 33, 13, 50),
    ("syn_2x", 65, 33, 13, 50),
]


def digest(row_ptr, col_idx):
    h = hashlib.sha256()
    h.update(struct.pack("<%di" % len(row_ptr), *row_ptr))
    h.update(struct.pack("<%di" % len(col_idx), *col_idx))
    return h.hexdigest()


def lines():
    out = []
    for name, T, C, W, n in SHAPES:
        for flags in (om.ROT_MOD_TPER, om.ROT_MOD_T, om.FIXED_GRID, om.WINDOW_ONLY):
            for s in range(n):
                rp, ci, _ = om.build_mask(T, C, W, s, flags)
                out.append(f"{name} {T} {C} {W} {flags} {s} {digest(rp, ci)}")
    return out


if __name__ == "__main__":
    with open(os.path.join(HERE, "mask_digests.txt"), "w") as f:
        f.write("# name T C W flags step sha256(int32le row_ptr ++ col_idx); written by gen_mask_digests.py from oracle/\n")
        f.write("\n".join(lines()) + "\n")
