"""Readers for the text fixtures under tests/golden/."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def q4_blocks():
    """Yield (name, block bytes uint8[18], expected binary16 bits uint16[32])."""
    name = block = None
    with open(os.path.join(GOLDEN, "q4_blocks.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, rest = line.partition(" ")
            if key == "name":
                name = rest
            elif key == "block":
                block = np.array([int(t, 16) for t in rest.split()], dtype=np.uint8)
                assert block.size == 18
            elif key == "expect":
                want = np.array([int(t, 16) for t in rest.split()], dtype=np.uint16)
                assert want.size == 32
                yield name, block, want
                name = block = None


def page_figures():
    """Key/value pairs of figures printed on the pages (tests/golden/page_figures.txt)."""
    out = {}
    with open(os.path.join(GOLDEN, "page_figures.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split("=", 1)
            out[k.strip()] = float(v.split("#")[0])
    return out
