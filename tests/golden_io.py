"""Reader for the hand-worked fixtures under tests/golden/."""

import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_blocks(name="mxfp4_blocks.txt"):
    blocks = {}
    extra = {}
    cur = None
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, rest = line.partition(" ")
            if key == "block":
                cur = blocks.setdefault(rest, {})
            elif key == "in":
                cur["in"] = np.array([float(v) for v in rest.split()], dtype=np.float64)
            elif key == "scale":
                cur["scale"] = int(rest, 16)
            elif key == "codes":
                cur["codes"] = np.array([int(v, 16) for v in rest.split()], dtype=np.uint8)
            else:
                extra[key] = rest
    return blocks, extra


def read_fp8(name="fp8_e4m3.txt"):
    """Hand-worked E4M3 values, rows and layout offsets (see the file's header)."""
    values, rows, layout = {}, [], None
    cur = None
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, rest = line.partition(" ")
            if key == "value":
                code, val = rest.split()
                values[int(code, 16)] = float(val)
            elif key == "row":
                name_, rs = rest.split()
                cur = {"name": name_, "round_scale": bool(int(rs))}
                rows.append(cur)
            elif key == "in":
                cur["in"] = np.array([float(v) for v in rest.split()], dtype=np.float64)
            elif key == "codes":
                cur["codes"] = np.array([int(v, 16) for v in rest.split()], dtype=np.uint8)
            elif key == "scale":
                cur["scale"] = bytes(int(v, 16) for v in rest.split())
            elif key == "layout":
                layout = tuple(int(v) for v in rest.split())
    return values, rows, layout
