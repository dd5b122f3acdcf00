"""Readers for the text fixtures under tests/golden/."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for ln in f:
            ln = ln.strip()
            if ln and not ln.startswith("#"):
                yield ln


def keyed_blocks(name, keys):
    """Blocks of 'key: values' lines, one block per len(keys) consecutive lines."""
    block = {}
    for ln in _lines(name):
        k, v = ln.split(":", 1)
        block[k.strip()] = v.split()
        if len(block) == len(keys):
            assert list(block) == list(keys), block
            yield block
            block = {}
    assert not block


def table(name):
    return [ln.split() for ln in _lines(name)]


def parse_float(s):
    return float("nan") if s == "nan" else float(s)


def sparse_row(tokens, K, dtype=np.float64):
    row = np.zeros(K, dtype)
    for t in tokens:
        i, v = t.split(":")
        row[int(i)] = float(v)
    return row
