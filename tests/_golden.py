"""Reader for the hand-derived stream fixtures under tests/golden/."""
import os

import numpy as np

GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    spec = {"bytes": {}}
    values = None
    for line in open(os.path.join(GOLDEN_DIR, name)):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        key, *rest = line.split()
        if key == "dtype":
            spec["dtype"] = {"bf16": 1, "e5m2": 2}[rest[0]]
        elif key == "input":
            values = [int(t, 16) for t in rest]
        elif key == "fill":
            values = [int(rest[1], 16)] * int(rest[0])
        elif key == "set":
            values[int(rest[0])] = int(rest[1], 16)
        elif key in ("codebook", "given_codebook"):
            spec[key] = bytes(int(t, 16) for t in rest)
        elif key in ("escapes", "size"):
            spec[key] = int(rest[0])
        elif key == "byte":
            spec["bytes"][int(rest[0])] = int(rest[1], 16)
        else:
            raise ValueError(f"unknown key {key} in {name}")
    spec["input"] = np.array(values, np.uint16 if spec["dtype"] == 1 else np.uint8)
    return spec


def names():
    """The exponent-codec fixtures (the lc_*.txt ones belong to the LC-style codec)."""
    return sorted(f for f in os.listdir(GOLDEN_DIR) if f.endswith(".txt") and not f.startswith("lc_"))
