"""Readers for the text fixtures under tests/golden/."""
import json
import os
import struct

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def f32(tok):
    """Parse a decimal / 'inf' / 'nan' / '-0' token or a '0x' bit pattern."""
    if tok.startswith("0x"):
        return struct.unpack("<f", struct.pack("<I", int(tok, 16)))[0]
    return float(tok)


def array(rows, dtype):
    if dtype == "f32":
        return np.array([[f32(t) for t in r] for r in rows], dtype=np.float32)
    return np.array([[int(t) for t in r] for r in rows], dtype=np.int32)


def nested(vals, dtype):
    def conv(v):
        if isinstance(v, list):
            return [conv(x) for x in v]
        return f32(v) if dtype == "f32" else int(v)
    return np.array(conv(vals), dtype=np.float32 if dtype == "f32" else np.int32)


def bits(a):
    """View a float32/int32 array as its raw int32 bit patterns."""
    return np.ascontiguousarray(a).view(np.int32)
