"""Reader for the small text fixtures under tests/golden/.

Format: '#' comment lines (the citation), then 'key value' lines, and blocks
introduced by a bare keyword ('input', 'output', 'output_first8') followed by
rows of whitespace-separated numbers until the next keyword.
"""
from __future__ import annotations

import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
_BLOCKS = {"input", "output", "output_first8"}


def load(name: str) -> dict:
    meta: dict = {}
    block = None
    with open(os.path.join(GOLDEN, name)) as f:
        for raw in f:
            line = raw.strip()
            if not line or line.startswith("#"):
                continue
            if line in _BLOCKS:
                block = line
                meta[block] = []
                continue
            head = line.split()[0]
            try:
                float(head)
                is_num = True
            except ValueError:
                is_num = False
            if is_num and block is not None:
                meta[block].append([float(v) for v in line.split()])
            else:
                key, _, value = line.partition(" ")
                meta[key] = value.strip()
                block = None
    for b in _BLOCKS & meta.keys():
        meta[b] = np.array(meta[b], dtype=np.float64)
    return meta
