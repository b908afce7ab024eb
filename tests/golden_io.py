"""Readers for the hand-written fixtures under tests/golden/."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if line:
                yield line


def codebook():
    vals = [int(v) for line in _lines("iq4_xs_codebook.txt") for v in line.split()]
    assert len(vals) == 16
    return np.array(vals, dtype=np.int64)


def hand_blocks():
    """{fmt_name: {"hex": bytes, field: [values] ...}}"""
    out, cur, key = {}, None, None
    for line in _lines("blocks_hand.txt"):
        if line.startswith("[") and line.endswith("]"):
            cur = out.setdefault(line[1:-1], {"hex": b""})
            key = None
            continue
        if ":" in line:
            k, v = line.split(":", 1)
            key = k.strip()
            if key != "hex":
                cur[key] = [float(t) for t in v.split()]
                key = None
            continue
        if key == "hex":
            cur["hex"] += bytes(int(t, 16) for t in line.split())
    return out


def act_cases():
    cases, cur = [], None
    for line in _lines("q8_act_cases.txt"):
        k, v = line.split(":", 1)
        vals = v.split()
        if k == "x":
            cur = {"x": np.zeros(32, np.float32)}
            cur["x"][: len(vals)] = np.array([float(t) for t in vals], np.float32)
            cases.append(cur)
        elif k == "q":
            cur["q"] = np.zeros(32, np.int64)
            cur["q"][: len(vals)] = [int(t) for t in vals]
        elif k == "d":
            cur["d"] = float(vals[0])
        elif k == "s":
            cur["s"] = int(vals[0])
    return cases
